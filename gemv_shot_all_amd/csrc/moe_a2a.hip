// moe_a2a.hip -- a mixture-of-experts down-projection fused with the combine
// all-to-all, at one rank's share, for gfx950.
//
// Rank `rank` holds ne experts.  A workgroup owns local expert e and TPW
// consecutive 16-feature tiles t0 .. t0 + TPW - 1.  Inside one launch it
//   a. reads the expert's split table (one segment per source rank), checks
//      it, and lays out its M <= GSA_MOE_MAX_TOKENS tokens: token j's row in X
//      and the row of its source rank's combine buffer that receives it;
//   b. for each tile of 16 tokens (the B operand's 16 columns): copies the
//      tokens' rows of X into LDS (each compute wave its own k-slice,
//      straight from memory with LDS DMA) and streams each feature tile's
//      16 weight rows with v_mfma_f32_16x16x32_bf16 (weights as the A
//      operand, tokens as the B operand, fp32 accumulation), the waves'
//      partials summed in wave order -- the weights of a later token tile
//      come back from L2, where the first one left them;
//   c. stores each token's results into its source rank's combine buffer,
//      waits for the stores, raises flag (rank, e, t) of each tile in every
//      rank's pad, and waits (bounded) for flag (p, e, t) of every other
//      rank p in its own pad.
//
// Sources (restated): a GEMM fused with an All-to-All for mixture-of-
// experts models, each workgroup handing its finished results to the
// collective at once and writing them straight into the destination's
// memory -- "Overlapping Collective Communication with Dependent Computation
// ... GPU-Initiated Intra-Kernel Networking", Abstract.  The dispatch layout
// (expert-major, source ranks in order, splits and offsets on the device)
// and the combine back to the source ranks -- "PyTorch Symmetric Memory"
// documentation, op reference of all_to_all_vdev_2d and
// all_to_all_vdev_2d_offset.  fp32 accumulation of bf16 -- same
// documentation, higher-precision reduction.
//
// Memory ordering as in the GEMV kernels: result rows and flags are
// agent-scope (sc1) accesses; every result store of the workgroup completes
// (s_waitcnt vmcnt(0), then a barrier) before its flags are stored.

#include <type_traits>

#include "gsa_device.h"
#include "gsa_internal.h"

namespace gsa {
namespace {

constexpr int kTok = 16;                     // tokens per MFMA tile: the B operand's 16 columns
constexpr int kMaxTok = GSA_MOE_MAX_TOKENS;  // tokens one local expert takes per call
constexpr int kWaves = 4;                    // compute waves per workgroup
// Largest chunks per row (F / 8) for which two token tiles of x and the
// partials of four feature tiles fit in 80 KB of LDS.
constexpr int kTwoTileMaxC = (80 * 1024 - (kWaves * 256 * 4 + 256 * 4) * 4) / (2 * 16 * 16) - 1;
static_assert(kMaxTok % kTok == 0, "whole token tiles");

__device__ __forceinline__ uint32_t* moe_flag(const MoeArgs& a, int pad, int src, int e, int t) {
  return a.pads + (int64_t)pad * a.pad_words + GSA_PAD_HEADER_WORDS +
         (int64_t)(src * a.ne + e) * a.row_stride + t;
}

// Every other rank's flag (p, e, t0 + q) in the own pad >= the tile's epoch
// for the nt tiles of a workgroup (lane 8 q + p), bounded by the timeout; on
// expiry the smallest missing (tile, rank) is recorded (wave 0 only).
__device__ void moe_wait_peers(const MoeArgs& a, int lane, int e, int t0, int nt,
                               const uint32_t* epochs) {
  uint32_t* own_pad = a.pads + (int64_t)a.rank * a.pad_words;
  const uint64_t start = wall_clock64();
  const int q = min(lane >> 3, nt - 1);   // lane 8 q + p: tile t0 + q, peer p
  const int p = min(lane & 7, a.W - 1);
  const int t = t0 + q;
  const uint32_t epoch = epochs[q];
  for (;;) {
    const uint32_t f = __hip_atomic_load(moe_flag(a, a.rank, p, e, t),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool lane_ok = (lane >> 3) >= nt || (lane & 7) >= a.W || p == a.rank || f >= epoch;
    const uint64_t missing = __ballot(!lane_ok);
    if (missing == 0) return;
    if (wall_clock64() - start > a.timeout_ticks) {
      if (lane == 0) {
        const uint32_t bit = (uint32_t)(__ffsll((long long)missing) - 1);
        atomicOr(own_pad + kHdrErrorBits, kErrTimeout);
        atomicMin(own_pad + kHdrTimeoutKey, (uint32_t)(e * a.tiles + t0 + (int)(bit >> 3)) * 8u + (bit & 7u));
      }
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// LDS (dynamic): x [16 NTT][C + 1] chunks (column C and rows past the
// tokens zero), the waves' 16 x (16 TPW) partials, the results token-major
// [16][16 TPW].  TPW: 16-feature tiles per workgroup (each x chunk read from
// LDS serves TPW MFMAs); RING: weight steps in flight per lane; NTT: token
// tiles one pass of the weights serves (each weight operand feeds NTT MFMAs).
template <int TPW, int RING, int NTT>
__global__ __launch_bounds__(kWaves * 64) void moe_gemm_a2a(MoeArgs a) {
  extern __shared__ uint4 lds[];
  __shared__ int64_t s_xrow[kMaxTok];  // token j: its row of X
  __shared__ int64_t s_dst[kMaxTok];   // token j: first element of its combine row
  __shared__ uint32_t s_ctl[4];     // -, ok, M
  __shared__ uint32_t s_ep[TPW];    // epoch of each tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int groups = (a.tiles + TPW - 1) / TPW;
  const int e = (int)(blockIdx.x / (unsigned)groups);
  const int t0 = (int)(blockIdx.x % (unsigned)groups) * TPW;
  const int nt = min(TPW, a.tiles - t0);
  const int C = a.C;
  const int CP = C + 1;  // padded LDS row: the 16 token rows of one chunk hit distinct banks
  float* red = reinterpret_cast<float*>(lds + NTT * 16 * CP);
  float* yt = red + kWaves * 256 * TPW;
  uint32_t* own_pad = a.pads + (int64_t)a.rank * a.pad_words;

  if (wave == 0) {
    // Lane s < W: source rank s's segment (every lane reads a valid entry).
    const int s = min(lane, a.W - 1);
    const int64_t len = a.splits[e * a.W + s];
    const int64_t ioff = a.splits[(int64_t)a.ne * a.W + e * a.W + s];
    const int64_t doff = a.dst_off[(int64_t)s * a.ne + e];
    const bool bad = lane < a.W && (len < 0 || ioff < 0 || doff < 0 || len > kMaxTok ||
                                    ioff + len > a.rows_in || doff + len > a.rows_out);
    const int mine = (lane < a.W && !bad) ? (int)len : 0;
    int before = 0, M = 0;  // rows of the lanes below this one, and in total
    for (int r = 0; r < a.W; ++r) {
      const int lr = __builtin_amdgcn_readlane(mine, r);
      before += r < lane ? lr : 0;
      M += lr;
    }
    const bool splits_ok = __ballot(bad) == 0 && M <= kMaxTok;
    const uint32_t own = __hip_atomic_load(moe_flag(a, a.rank, a.rank, e, t0 + min(lane, nt - 1)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // tiles whose own flag row is marked published or has its epochs exhausted
    const uint64_t own_bad = __ballot(lane < nt && own >= GSA_FLAG_PUBLISHED - 1u);
    const bool own_ok = own_bad == 0;
    if (splits_ok && own_ok && lane < a.W) {
      for (int i = 0; i < mine; ++i) {
        s_xrow[before + i] = ioff + i;
        s_dst[before + i] = ((int64_t)lane * a.rows_out + doff + i) * a.H;
      }
    }
    if (lane < nt) s_ep[lane] = own + 1u;
    if (lane == 0) {
      if (!splits_ok) {
        atomicOr(own_pad + kHdrErrorBits, kErrSplit);
        atomicMin(own_pad + kHdrSplitExpert, (uint32_t)e);
      }
      if (!own_ok) {
        atomicOr(own_pad + kHdrErrorBits, kErrState);
        atomicMin(own_pad + kHdrStateTile,
                  (uint32_t)(e * a.tiles + t0 + __ffsll((long long)own_bad) - 1));
      }
      s_ctl[1] = (splits_ok && own_ok) ? 1u : 0u;
      s_ctl[2] = (uint32_t)M;
    }
  }
  __syncthreads();  // B0: token table and decision in LDS
  if (s_ctl[1] == 0u) return;
  const int M = (int)s_ctl[2];

  if (M > 0) {
    const int steps = (C + 3) / 4;
    const int per_wave = (steps + kWaves - 1) / kWaves;
    const int s_begin = wave * per_wave;
    const int n_steps = max(0, min(steps, s_begin + per_wave) - s_begin);
    const int c_begin = min(4 * s_begin, C);
    const int c_end = min(4 * (s_begin + n_steps), C);

    const uint4* xg = reinterpret_cast<const uint4*>(a.X);
    const uint16_t* w_e = a.Wd + (int64_t)e * a.H * a.F;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(w_e, (uint32_t)(a.H * a.F * 2));
    const int kq = lane >> 4;
    const uint32_t a_row = ((uint32_t)(t0 * 16 + (lane & 15)) * (uint32_t)C + kq) * 16u;
    const uint32_t tile_bytes = 16u * (uint32_t)C * 16u;
    // Weights with the default cache policy: an MFMA operand load reads 64
    // bytes (half a 128-byte line) of each of 16 rows, and the next step
    // reads the other halves; without the non-temporal hint those lines are
    // still in L2 when it asks (measured 204 -> 182 us on the DeepSeek-V3-like
    // shape, 17.0 -> 16.6 us on the Qwen3-30B-A3B-like one), and a second
    // token tile finds them there too.
    const uint32_t kOutOfRange = 0x80000000u;  // past any weight: reads zeros
    auto a_off = [&](int j, int q) {
      return j < n_steps ? a_row + (uint32_t)q * tile_bytes + (uint32_t)(s_begin + j) * 64u : kOutOfRange;
    };
    const int xrow = (lane & 15) * CP;
    const int j = tid >> 4;  // the store phase: token j of the tile, feature n of each feature tile
    const int n = tid & 15;

    // One pass of the weights over NT token tiles (tokens jt .. jt + 16 NT - 1,
    // tile u in LDS rows 16 u ..): every weight operand feeds NT MFMAs, so the
    // expert's weights are streamed once per NT tiles.  Each wave reads only
    // its own k-slice of the rows (and the zero column C), so no barrier
    // guards them; the partials' buffers are guarded by B1 / B2.
    auto pass = [&](auto nt_const, int jt) {
      constexpr int NT = decltype(nt_const)::value;
      int mt[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) mt[u] = max(0, min(kTok, M - jt - u * kTok));
      for (int c0 = c_begin; c0 < c_end; c0 += 64) {
        if (c0 + lane < c_end) {
#pragma unroll
          for (int u = 0; u < NT; ++u)
            for (int t = 0; t < mt[u]; ++t)
              lds_dma16(xg + s_xrow[jt + u * kTok + t] * C + c0 + lane,
                        lds + (u * kTok + t) * CP + c0);
        }
      }
      uint4 ring[RING][TPW];
#pragma unroll
      for (int u = 0; u < RING; ++u)
#pragma unroll
        for (int q = 0; q < TPW; ++q) ring[u][q] = buf_load16_cached(ra, a_off(u, q));
      // The x copies went out before the ring loads: once at most RING * TPW
      // loads are outstanding they have landed.
      wait_vm_le<RING * TPW>();
#pragma unroll
      for (int u = 0; u < NT; ++u)
        for (int c = c_begin + lane; c < c_end; c += 64)
          for (int t = mt[u]; t < kTok; ++t) lds[(u * kTok + t) * CP + c] = make_uint4(0u, 0u, 0u, 0u);
      if (lane < NT * kTok) lds[lane * CP + C] = make_uint4(0u, 0u, 0u, 0u);

      f32x4_t acc[TPW][NT];
#pragma unroll
      for (int q = 0; q < TPW; ++q)
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[q][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      for (int j0 = 0; j0 < n_steps; j0 += RING) {
        uint4 xv[RING][NT];
#pragma unroll
        for (int u = 0; u < RING; ++u) {
          const int js = j0 + u;
          const int chunk = 4 * (s_begin + js) + kq;
#pragma unroll
          for (int v = 0; v < NT; ++v)
            xv[u][v] = lds[v * kTok * CP + xrow + (js < n_steps && chunk < C ? chunk : C)];
        }
#pragma unroll
        for (int u = 0; u < RING; ++u) {
#pragma unroll
          for (int q = 0; q < TPW; ++q) {
#pragma unroll
            for (int v = 0; v < NT; ++v)
              acc[q][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, ring[u][q]), __builtin_bit_cast(bf16x8_t, xv[u][v]),
                  acc[q][v], 0, 0, 0);
            ring[u][q] = buf_load16_cached(ra, a_off(j0 + u + RING, q));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int v = 0; v < NT; ++v) {
        // Partials: feature 4 * (lane >> 4) + q, token lane & 15.
        // red[wave][q*16 + feature][token]
#pragma unroll
        for (int q = 0; q < TPW; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[(wave * 16 * TPW + q * 16 + 4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[q][v][r];
        __syncthreads();  // B1
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
          const int nl = q * 16 + 4 * wave + (lane >> 4);
          const int bl = lane & 15;
          float y = red[nl * 16 + bl];
#pragma unroll
          for (int w = 1; w < kWaves; ++w) y = y + red[(w * 16 * TPW + nl) * 16 + bl];
          yt[bl * 16 * TPW + nl] = y;
        }
        __syncthreads();  // B2: results token-major (and red free again)
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
          const int64_t feat = (int64_t)(t0 + q) * 16 + n;
          if (j < mt[v] && q < nt && feat < a.H)
            store_coherent(&a.bufs[s_dst[jt + v * kTok + j] + feat], yt[j * 16 * TPW + q * 16 + n]);
        }
      }
    };
    // Two token tiles per pass where the launch staged room for them and
    // more than one tile's tokens remain; one otherwise.
    for (int jt = 0; jt < M;) {
      if (NTT >= 2 && M - jt > kTok) {
        pass(std::integral_constant<int, (NTT >= 2 ? 2 : 1)>{}, jt);
        jt += (NTT >= 2 ? 2 : 1) * kTok;
      } else {
        pass(std::integral_constant<int, 1>{}, jt);
        jt += kTok;
      }
    }
  }
  wait_vm_all();    // this wave's result rows are at the coherence point ...
  __syncthreads();  // B3 ... in every wave
  if (wave == 0) {
    // lane 8 q + d: tile t0 + q's flag in pad d
    if ((lane >> 3) < nt && (lane & 7) < a.W)
      store_flag(moe_flag(a, lane & 7, a.rank, e, t0 + (lane >> 3)), s_ep[lane >> 3]);
    moe_wait_peers(a, lane, e, t0, nt, s_ep);
  }
}

__global__ void a2a_reset_kernel(uint32_t* pads, int ne, int row_stride, int64_t pad_words,
                                 int64_t total, uint32_t mask) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t w = i % pad_words;  // word within its pad
  uint32_t v;
  if (w < GSA_PAD_HEADER_WORDS) {
    v = (w == kHdrTimeoutKey || w == kHdrStateTile || w == kHdrEpiWaitTile ||
         w == kHdrSplitExpert)
            ? 0xFFFFFFFFu
            : 0u;
  } else {
    const int src = (int)((w - GSA_PAD_HEADER_WORDS) / row_stride) / ne;
    v = ((mask >> src) & 1u) ? GSA_FLAG_PUBLISHED : 0u;
  }
  pads[i] = v;
}

}  // namespace

namespace {

template <int TPW, int NTT>
size_t lds_bytes(int C) {
  return (size_t)16 * NTT * (C + 1) * 16 +
         (size_t)(kWaves * 256 * TPW + 256 * TPW) * sizeof(float);
}

template <int TPW, int RING, int NTT>
hipError_t launch(const MoeArgs& a, hipStream_t s) {
  const size_t lds = lds_bytes<TPW, NTT>(a.C);
  if (lds > 65536) {
    // Opt in to the largest dynamic LDS this instance may use (cheap, idempotent).
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_a2a<TPW, RING, NTT>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)lds_bytes<TPW, NTT>(NTT > 1 ? kTwoTileMaxC : GSA_MOE_MAX_F / 8));
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)(a.ne * ((a.tiles + TPW - 1) / TPW));
  hipLaunchKernelGGL((moe_gemm_a2a<TPW, RING, NTT>), dim3(grid), dim3(kWaves * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// Tiles per workgroup by the width F of the expert: narrow experts take four
// 16-feature tiles per workgroup, wide ones two, so that each workgroup
// streams about 100-130 KB of weights and its fixed costs (split table, token
// staging, store acknowledgement, flags) are spread over more bytes.
// Measured on the Qwen3-30B-A3B-like (F = 768) and DeepSeek-V3-like
// (F = 2048) shapes: one tile per workgroup 21.7 / 236 us, two 18.7 / 205,
// four 17.0 / 230.
//
// Experts narrow enough that two token tiles of x stay within 80 KB of LDS
// with the partials (two workgroups per CU) take two token tiles per pass of
// their weights: an expert with more than 16 tokens streams its weights half
// as often (the host does not know the token counts, which live on the
// device; an expert with at most 16 takes the one-tile pass, at the price of
// the second tile's LDS).
hipError_t launch_moe(const MoeArgs& a, hipStream_t s) {
  if (a.F > 1024) return launch<2, 8, 1>(a, s);
  return a.C <= kTwoTileMaxC ? launch<4, 4, 2>(a, s) : launch<4, 4, 1>(a, s);
}

hipError_t launch_a2a_reset(uint32_t* pads, int W, int ne, int row_stride, int64_t pad_words,
                            uint32_t published_mask, hipStream_t s) {
  const int64_t total = (int64_t)W * pad_words;
  const unsigned block = 256;
  const unsigned grid = (unsigned)((total + block - 1) / block);
  hipLaunchKernelGGL(a2a_reset_kernel, dim3(grid), dim3(block), 0, s, pads, ne, row_stride,
                     pad_words, total, published_mask);
  return hipGetLastError();
}

}  // namespace gsa
