// gemv_allreduce.hip -- the fused GEMV + one-shot AllReduce kernels for gfx950.
//
// One workgroup owns one flag tile: 16 output rows x all B batch columns.
// Inside one launch it
//   a. reads its own flag (epoch e = flag + 1) and polls the peers' flags
//      for its tile; if every peer has already published (always the case
//      for simulated peers) it acquires and prefetches the peer slots so
//      their latency hides under the A stream;
//   b. stages this rank's activation slice x (bf16) in LDS;
//   c. streams its 16 rows of A_r with 128-bit loads and multiply-adds in
//      fp32 (VALU bf16 dot2 for B <= 8, MFMA 16x16x32 for 8 < B <= 16);
//   d. reduces lane partials with a fixed butterfly (or, for MFMA, a fixed
//      cross-wave sum through LDS);
//   e. publishes y into slot[rank], releases flag[rank][tile] = e, waits (if
//      step a did not already see them) for every peer's flag >= e, and
//      writes out = ((0 + s_0) + s_1) ... + s_{W-1} in rank order.
//
// Sources (restated): fused GEMV + AllReduce with per-workgroup hand-off of
// finished results -- "Overlapping Collective Communication with Dependent
// Computation ... GPU-Initiated Intra-Kernel Networking", Abstract.  One-shot
// sum over all ranks' buffers in rank order from zero, signal pad indexed by
// block -- "PyTorch Symmetric Memory" documentation, writing-your-own-kernel
// section and the multimem_all_reduce_ warning in the op reference.
// fp32 accumulation of bf16 -- same documentation, higher-precision reduction.
//
// No value atomics and fixed reduction trees: repeated calls are bit-identical.

#include "gsa_internal.h"

namespace gsa {
namespace {

constexpr int kTileRows = GSA_FLAG_TILE_ROWS;
constexpr int kMaxW = GSA_MAX_W;

// s_ctl[1] values: what the start-of-kernel poll found.
enum : uint32_t { kMustWait = 0u, kPeersReady = 1u, kBadOwnRow = 2u };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// acc += <8 bf16 of a, 8 bf16 of x>, as four fp32 dot2 steps in k order.
__device__ __forceinline__ float dot8(const uint4& a, const uint4& x, float acc) {
  acc = dot2(a.x, x.x, acc);
  acc = dot2(a.y, x.y, acc);
  acc = dot2(a.z, x.z, acc);
  acc = dot2(a.w, x.w, acc);
  return acc;
}

__device__ __forceinline__ uint32_t* flag_ptr(const GemvArgs& a, int r, int64_t t) {
  return a.pad + GSA_PAD_HEADER_WORDS + (int64_t)r * a.row_stride + t;
}

// Lane p reads flag[min(p, W-1)][t] (no divergent loads: every lane reads a
// valid word; lanes >= W are ignored by the callers).
__device__ __forceinline__ uint32_t load_flag(const GemvArgs& a, int lane, int64_t t) {
  return __hip_atomic_load(flag_ptr(a, min(lane, a.W - 1), t), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Rank r's 16 x B tile of slot r lands at pe[(r * 16 + n) * B + b].  Rows
// past N are clamped (their values are never used).  Every lane issues all
// its loads before the first LDS write (ranks >= W are clamped to W-1 and
// written to the sink at pe[W * 16 * B]).
__device__ __forceinline__ void load_peer_tile(const GemvArgs& a, int lane, int64_t tile,
                                               float* pe) {
  const int64_t NB = a.N * a.B;
  const int tb = kTileRows * a.B;                // elements of one rank's tile
  const int64_t first = tile * kTileRows * a.B;  // first element of the tile in a slot
  const int64_t last = NB - 1;
  constexpr int kPerLane = (kTileRows * GSA_MAX_B) / 64;  // 4
  float v[kMaxW][kPerLane];
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) {
    const float* src = a.slots + min(r, a.W - 1) * NB;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) v[r][i] = src[min(first + lane + 64 * i, last)];
  }
  const int sink = a.W * tb;
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + 64 * i;
      pe[(r < a.W && e < tb) ? r * tb + e : sink] = v[r][i];
    }
  }
}

// The communication wave's part before the workgroup's second barrier: derive
// the epoch from its own flag, check every peer's flag for this tile, and if
// all have published, acquire and copy the peers' tiles into LDS.  Writes
// s_ctl[0] = epoch and s_ctl[1] = kMustWait / kPeersReady / kBadOwnRow.
__device__ __forceinline__ void comm_start(const GemvArgs& a, int lane, int64_t tile,
                                           uint32_t fl, float* pe, uint32_t* s_ctl) {
  const uint32_t own = __builtin_amdgcn_readlane(fl, a.rank);
  if (own >= GSA_FLAG_PUBLISHED - 1u) {  // row marked published, or epochs exhausted
    if (lane == 0) {
      atomicOr(a.pad + kHdrErrorBits, kErrState);
      atomicMin(a.pad + kHdrStateTile, (uint32_t)tile);
      s_ctl[1] = kBadOwnRow;
    }
    return;
  }
  const uint32_t epoch = own + 1u;
  const bool lane_ok = lane >= a.W || lane == a.rank || fl >= epoch;
  const bool ready = __ballot(!lane_ok) == 0;
  if (ready) {
    acquire_fence();
    load_peer_tile(a, lane, tile, pe);
  }
  if (lane == 0) {
    s_ctl[0] = epoch;
    s_ctl[1] = ready ? kPeersReady : kMustWait;
  }
}

// Bounded wait for every peer's flag >= epoch.  On expiry records the
// smallest missing peer of this tile in the pad header.
__device__ bool wait_peers(const GemvArgs& a, int lane, int64_t tile, uint32_t epoch) {
  const uint64_t start = wall_clock64();
  for (;;) {
    const uint32_t f = load_flag(a, lane, tile);
    const bool lane_ok = lane >= a.W || lane == a.rank || f >= epoch;
    const uint64_t missing = __ballot(!lane_ok);
    if (missing == 0) {
      acquire_fence();
      return true;
    }
    if (wall_clock64() - start > a.timeout_ticks) {
      if (lane == 0) {
        const uint32_t peer = (uint32_t)(__ffsll((long long)missing) - 1);
        atomicOr(a.pad + kHdrErrorBits, kErrTimeout);
        atomicMin(a.pad + kHdrTimeoutKey, (uint32_t)tile * 8u + peer);
      }
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The communication wave (the last wave of every workgroup).  It does the
// signal-pad protocol so that its waits never hold up the A stream of the
// compute waves.  Barrier schedule shared with the compute waves:
//   B1 x staged | B2 partials + peer tile ready | B3 own slot published
//   | B4 (only if the peers were not ready at B2) late peer tile ready.
__device__ void comm_wave(const GemvArgs& a, int lane, int64_t tile, float* pe,
                          uint32_t* s_ctl) {
  const uint32_t fl = load_flag(a, lane, tile);
  __syncthreads();  // B1
  comm_start(a, lane, tile, fl, pe, s_ctl);
  __syncthreads();  // B2
  const uint32_t state = s_ctl[1];
  if (state == kBadOwnRow) return;
  const uint32_t epoch = s_ctl[0];
  __syncthreads();  // B3: the compute waves' slot stores precede this barrier
  if (lane == 0)
    __hip_atomic_store(flag_ptr(a, a.rank, tile), epoch, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (state == kPeersReady) return;
  const bool ok = wait_peers(a, lane, tile, epoch);
  if (ok) load_peer_tile(a, lane, tile, pe);
  if (lane == 0) s_ctl[1] = ok ? kPeersReady : kMustWait;
  __syncthreads();  // B4
}

// out = ((0 + s_0) + s_1) ... + s_{W-1}; s_rank is this call's published y,
// the others come from the peer tile in LDS (local row n, column b).
__device__ __forceinline__ float one_shot_sum(const GemvArgs& a, float y, const float* pe, int n,
                                              int b) {
  const int tb = kTileRows * a.B;
  float acc = 0.0f;
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) {
    if (r < a.W) acc = acc + (r == a.rank ? y : pe[r * tb + n * a.B + b]);
  }
  return acc;
}

// Compute waves once their partials are final and barrier B2 has passed
// (y[e] for local rows n[e], column b, owner lanes only): publish, (reduce),
// B3, [B4, reduce].
template <int OPL>
__device__ void finish_after_b2(const GemvArgs& a, int64_t tile, const int (&n)[OPL], int b,
                                const bool (&live)[OPL], const float (&y)[OPL], const float* pe,
                                const uint32_t* s_ctl) {
  const uint32_t state = s_ctl[1];
  if (state == kBadOwnRow) return;
  const int64_t NB = a.N * a.B;
  const int64_t row0 = tile * kTileRows;
  float* own_slot = a.slots + a.rank * NB;
#pragma unroll
  for (int e = 0; e < OPL; ++e)
    if (live[e]) own_slot[(row0 + n[e]) * a.B + b] = y[e];
  if (state == kPeersReady) {
#pragma unroll
    for (int e = 0; e < OPL; ++e)
      if (live[e]) a.out[(row0 + n[e]) * a.B + b] = one_shot_sum(a, y[e], pe, n[e], b);
  }
  __syncthreads();  // B3
  if (state == kPeersReady) return;
  __syncthreads();  // B4
  if (s_ctl[1] != kPeersReady) return;  // wait expired: this tile's out rows stay unwritten
#pragma unroll
  for (int e = 0; e < OPL; ++e)
    if (live[e]) a.out[(row0 + n[e]) * a.B + b] = one_shot_sum(a, y[e], pe, n[e], b);
}

// MFMA epilogue: B2, wave 0 sums the compute waves' partials in wave order,
// then publishes and reduces.
template <int NW>
__device__ void mfma_finish(const GemvArgs& a, int64_t tile, int wave, int lane,
                            const int (&n)[4], int b, const bool (&live)[4], f32x4_t acc,
                            const float* red, const float* pe, const uint32_t* s_ctl) {
  __syncthreads();  // B2
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = acc[e];
  if (wave == 0) {
    for (int w = 1; w < NW; ++w) {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = y[e] + red[((w - 1) * 4 + e) * 64 + lane];
    }
  }
  finish_after_b2<4>(a, tile, n, b, live, y, pe, s_ctl);
}

// Butterfly reduction of P values over a group of G lanes (G, P powers of
// two, P <= G).  Each step halves the values a lane keeps and the lanes it
// spans; afterwards lane li holds the group total of value li / (G / P).
template <int G, int P>
__device__ __forceinline__ void butterfly(float* v, int li) {
  if constexpr (G > 1) {
    constexpr int OFF = G / 2;
    if constexpr (P > 1) {
      constexpr int H = P / 2;
      const bool up = (li & OFF) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, OFF);
      }
      butterfly<OFF, H>(v, li);
    } else {
      v[0] = v[0] + __shfl_xor(v[0], OFF);
      butterfly<OFF, 1>(v, li);
    }
  }
}

// A chunks [base + li + j*G] of rows rowc[0..R-1] (already clamped to N-1).
// MASKED: chunks past the row end are clamped to a valid chunk; mac_pass pairs
// them with a zero x chunk, so they add nothing (A is finite).
template <bool MASKED, int CPL, int R, int G>
__device__ __forceinline__ void load_a(uint4 (&av)[CPL][R], const uint4* Ag,
                                       const int64_t (&rowc)[R], int C, int li, int base) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + li + j * G;
    const int cc = MASKED ? min(c, C - 1) : c;
#pragma unroll
    for (int s = 0; s < R; ++s) av[j][s] = Ag[rowc[s] * C + cc];
  }
}

// x chunks live at lds_x[b * C + c]; lds_x[B * C] holds a zero chunk.
template <bool MASKED, int B, int R, int CPL, int G>
__device__ __forceinline__ void mac_pass(float (&acc)[R][B], const uint4 (&av)[CPL][R],
                                         const uint4* lds_x, int C, int li, int base) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + li + j * G;
    uint4 xv[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xv[b] = lds_x[(MASKED && c >= C) ? B * C : b * C + c];
#pragma unroll
    for (int s = 0; s < R; ++s)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[s][b] = dot8(av[j][s], xv[b], acc[s][b]);
  }
}

// Main loop of the VALU kernel: the first pass's A chunks are already in
// registers; later passes load and accumulate.
template <bool MASKED, int B, int G, int R, int CPL>
__device__ __forceinline__ void valu_passes(float (&acc)[R][B], uint4 (&av)[CPL][R],
                                            const uint4* Ag, const int64_t (&rowc)[R],
                                            const uint4* lds_x, int C, int li) {
  mac_pass<MASKED, B, R, CPL, G>(acc, av, lds_x, C, li, 0);
  for (int base = G * CPL; base < C; base += G * CPL) {
    load_a<MASKED, CPL, R, G>(av, Ag, rowc, C, li, base);
    mac_pass<MASKED, B, R, CPL, G>(acc, av, lds_x, C, li, base);
  }
}

// VALU path, B <= 8.  NW compute waves plus one communication wave.  Each
// compute wave holds 64/G row groups of R rows; a row group of G lanes walks
// one row in 16-byte chunks li, li+G, ...  CPL chunks per lane are loaded per
// pass (the first pass before the LDS barrier, behind the x loads); XPT x
// chunks per thread are staged through registers.  Chunk masking is only
// compiled into the branch taken when C is not a multiple of G * CPL.
// LDS: x chunks [b][c], one zero chunk, one sink chunk; then the peer tile.
template <int B, int G, int R, int NW, int CPL, int XPT>
__global__ __launch_bounds__((NW + 1) * 64) void gemv_ar_valu(GemvArgs a) {
  constexpr int NT = NW * 64;
  constexpr int GPW = 64 / G;
  static_assert(NW * GPW * R == kTileRows, "one workgroup covers one flag tile");
  constexpr int V = R * B;
  constexpr int P = pow2_ceil(V);
  static_assert(P <= G, "butterfly needs P <= G");

  extern __shared__ uint4 lds_x[];
  __shared__ uint32_t s_ctl[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const int C = a.C;
  const int xchunks = B * C;
  float* pe = reinterpret_cast<float*>(lds_x + xchunks + 2);

  if (wave == NW) {
    comm_wave(a, lane, tile, pe, s_ctl);
    return;
  }

  const int grp = lane / G;
  const int li = lane % G;
  const int nloc0 = (wave * GPW + grp) * R;  // first local row of this row group
  const int64_t row0 = tile * kTileRows + nloc0;
  const bool masked = (C % (G * CPL)) != 0;

  const uint4* xg = reinterpret_cast<const uint4*>(a.x);
  uint4 xr[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) xr[i] = xg[min(tid + i * NT, xchunks - 1)];

  const uint4* Ag = reinterpret_cast<const uint4*>(a.A);
  int64_t rowc[R];
#pragma unroll
  for (int s = 0; s < R; ++s) rowc[s] = min(row0 + s, a.N - 1);
  uint4 av[CPL][R];
  if (masked)
    load_a<true, CPL, R, G>(av, Ag, rowc, C, li, 0);
  else
    load_a<false, CPL, R, G>(av, Ag, rowc, C, li, 0);

#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int idx = tid + i * NT;
    lds_x[idx < xchunks ? idx : xchunks + 1] = xr[i];  // out-of-range lanes: sink
  }
  for (int idx = tid + XPT * NT; idx < xchunks; idx += NT) lds_x[idx] = xg[idx];
  if (tid == 0) lds_x[xchunks] = make_uint4(0u, 0u, 0u, 0u);  // zero chunk for masking
  __syncthreads();  // B1

  float acc[R][B];
#pragma unroll
  for (int s = 0; s < R; ++s)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[s][b] = 0.0f;
  if (masked)
    valu_passes<true, B, G, R, CPL>(acc, av, Ag, rowc, lds_x, C, li);
  else
    valu_passes<false, B, G, R, CPL>(acc, av, Ag, rowc, lds_x, C, li);

  float v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) v[i] = i < V ? acc[i / B][i % B] : 0.0f;
  butterfly<G, P>(v, li);

  // Lane li now holds value vidx = s * B + b of its row group.
  const int vidx = li / (G / P);
  const bool owner = (li % (G / P)) == 0 && vidx < V;
  const int n[1] = {nloc0 + min(vidx, V - 1) / B};
  const bool live[1] = {owner && tile * kTileRows + n[0] < a.N};
  const float y[1] = {v[0]};
  __syncthreads();  // B2
  finish_after_b2<1>(a, tile, n, vidx % B, live, y, pe, s_ctl);
}

// A operand chunks of k-steps s0..s0+SPW-1 for MFMA lane (row arowc, chunk
// group kq).  MASKED: indices are clamped to a valid chunk; mfma_pass pairs
// steps past s_end and chunks past the row with the zero x column.
template <bool MASKED, int SPW>
__device__ __forceinline__ void load_a_mfma(uint4 (&av)[SPW], const uint4* Ag, int64_t arowc,
                                            int C, int kq, int s0) {
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int chunk = 4 * (s0 + u) + kq;
    av[u] = Ag[arowc * C + (MASKED ? min(chunk, C - 1) : chunk)];
  }
}

// x chunk (batch xb, chunk c) at lds[xb * CP + c]; column C of every batch
// row is zero.
template <bool MASKED, int SPW>
__device__ __forceinline__ f32x4_t mfma_pass(f32x4_t acc, const uint4 (&av)[SPW],
                                             const uint4* lds, int CP, int C, int xb, int kq,
                                             int s0, int s_end) {
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int chunk = 4 * (s0 + u) + kq;
    const int cc = MASKED ? ((s0 + u < s_end && chunk < C) ? chunk : C) : chunk;
    const uint4 xv = lds[xb * CP + cc];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                  __builtin_bit_cast(bf16x8_t, xv), acc, 0, 0, 0);
  }
  return acc;
}

template <bool MASKED, int SPW>
__device__ __forceinline__ f32x4_t mfma_steps(uint4 (&av)[SPW], const uint4* Ag, int64_t arowc,
                                              const uint4* lds, int CP, int C, int xb, int kq,
                                              int s_begin, int s_end) {
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = s_begin; s0 < s_end; s0 += SPW) {
    if (s0 != s_begin) load_a_mfma<MASKED, SPW>(av, Ag, arowc, C, kq, s0);
    acc = mfma_pass<MASKED, SPW>(acc, av, lds, CP, C, xb, kq, s0, s_end);
  }
  return acc;
}

// MFMA path, 8 < B <= 16 (batch padded to 16 with zeros).  The tile's 16 rows
// form the A operand of v_mfma_f32_16x16x32_bf16, x (16 batches x 32 k) the
// B operand from LDS.  The NW compute waves split the k-steps; their 16x16
// fp32 partials are summed in wave order through LDS.  One more wave runs
// the signal-pad protocol.  Operand layout per lane l: A row (l & 15), B
// column (l & 15), k-chunk (l >> 4) of the step's four 8-element chunks;
// result rows 4*(l >> 4) + e, column (l & 15).
// LDS: x [16][C + 1] chunks (column C zero); (NW-1) x 4 x 64 partials; peer tile.
template <int NW, int SPW, int XC>
__global__ __launch_bounds__((NW + 1) * 64) void gemv_ar_mfma(GemvArgs a) {
  constexpr int NT = NW * 64;
  extern __shared__ uint4 lds[];
  __shared__ uint32_t s_ctl[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const int C = a.C;
  const int CP = C + 1;  // padded LDS row: spreads the 16 batch rows over banks
  float* red = reinterpret_cast<float*>(lds + 16 * CP);
  float* pe = red + (NW - 1) * 4 * 64;

  if (wave == NW) {
    comm_wave(a, lane, tile, pe, s_ctl);
    return;
  }

  const int64_t row0 = tile * kTileRows;
  const int steps = (C + 3) / 4;
  const int per_wave = (steps + NW - 1) / NW;
  const int s_begin = wave * per_wave;
  const int s_end = min(steps, s_begin + per_wave);
  const bool masked = (C % 4) != 0 || (steps % NW) != 0 || (per_wave % SPW) != 0;

  const uint4* xg = reinterpret_cast<const uint4*>(a.x);
  uint4 xr[XC][16];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = min(tid + i * NT, C - 1);
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      uint4 v = xg[min(b, a.B - 1) * C + c];
      if (b >= a.B) v = make_uint4(0u, 0u, 0u, 0u);
      xr[i][b] = v;
    }
  }

  const uint4* Ag = reinterpret_cast<const uint4*>(a.A);
  const int64_t arowc = min(row0 + (lane & 15), a.N - 1);
  const int kq = lane >> 4;
  uint4 av[SPW];
  if (masked)
    load_a_mfma<true, SPW>(av, Ag, arowc, C, kq, s_begin);
  else
    load_a_mfma<false, SPW>(av, Ag, arowc, C, kq, s_begin);

#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = tid + i * NT;
    if (c >= C) continue;
#pragma unroll
    for (int b = 0; b < 16; ++b) lds[b * CP + c] = xr[i][b];
  }
  for (int c = tid + XC * NT; c < C; c += NT) {
    for (int b = 0; b < 16; ++b)
      lds[b * CP + c] = b < a.B ? xg[b * C + c] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid < 16) lds[tid * CP + C] = make_uint4(0u, 0u, 0u, 0u);  // zero column
  __syncthreads();  // B1

  const int xb = lane & 15;
  f32x4_t acc;
  if (masked)
    acc = mfma_steps<true, SPW>(av, Ag, arowc, lds, CP, C, xb, kq, s_begin, s_end);
  else
    acc = mfma_steps<false, SPW>(av, Ag, arowc, lds, CP, C, xb, kq, s_begin, s_end);

  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave - 1) * 4 + e) * 64 + lane] = acc[e];
  }
  // B2 is inside compute_wave_finish; wave 0 reads the other partials after it.
  const int b_own = min(lane & 15, a.B - 1);
  int n[4];
  bool live[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    n[e] = 4 * (lane >> 4) + e;
    live[e] = wave == 0 && (lane & 15) < a.B && row0 + n[e] < a.N;
  }
  mfma_finish<NW>(a, tile, wave, lane, n, b_own, live, acc, red, pe, s_ctl);
}

__global__ void pad_reset_kernel(uint32_t* pad, int W, int row_stride, uint32_t mask) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = GSA_PAD_HEADER_WORDS + (int64_t)W * row_stride;
  if (i >= total) return;
  uint32_t v;
  if (i < GSA_PAD_HEADER_WORDS) {
    v = (i == kHdrTimeoutKey || i == kHdrStateTile) ? 0xFFFFFFFFu : 0u;
  } else {
    const int r = (int)((i - GSA_PAD_HEADER_WORDS) / row_stride);
    v = ((mask >> r) & 1u) ? GSA_FLAG_PUBLISHED : 0u;
  }
  pad[i] = v;
}

constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
constexpr int kMfmaWaves = 4;

struct ValuChoice {
  const void* kernel;
  int waves;  // compute waves (the communication wave comes on top)
};

// CMAX: largest C of the tier; XPT covers B * CMAX chunks (at most 8 per thread).
template <int B, int G, int R, int NW, int CPL, int CMAX>
ValuChoice valu_choice() {
  constexpr int XPT0 = ceil_div(B * CMAX, NW * 64);
  constexpr int XPT = XPT0 > 8 ? 8 : XPT0;
  return {reinterpret_cast<const void*>(&gemv_ar_valu<B, G, R, NW, CPL, XPT>), NW};
}

// VALU tiers by chunks per row C = Ks / 8 (every tier covers 16 rows per
// workgroup, plus the communication wave):
//   C <= 64 : 4 waves, a full wave per row, 4 rows per wave, 1 chunk per pass
//   C <= 224: 4 waves, half a wave per row, 2 x 2 rows per wave, 7 chunks
//   larger  : 8 waves, a full wave per row, 2 rows per wave, 7 chunks per
//             pass (4 for B > 4, to stay within 168 VGPRs)
template <int B>
ValuChoice valu_kernel(int C) {
  if (C <= 64) return valu_choice<B, 64, 4, 4, 1, 64>();
  if (C <= 224) return valu_choice<B, 32, 2, 4, 7, 224>();
  return valu_choice<B, 64, 2, 8, (B <= 4 ? 7 : 4), 448>();
}

}  // namespace

size_t gemv_lds_bytes(int W, int B, int C) {
  const size_t peer_tile = ((size_t)W * kTileRows * B + 1) * sizeof(float);
  if (B <= 8) return ((size_t)B * C + 2) * 16 + peer_tile;
  return (size_t)16 * (C + 1) * 16 + (size_t)(kMfmaWaves - 1) * 4 * 64 * sizeof(float) +
         peer_tile;
}

bool select_gemv_kernel(int W, int B, int C, Launch* out) {
  if (W < 1 || W > GSA_MAX_W || B < 1 || B > GSA_MAX_B || C < 1) return false;
  const size_t x_bytes = B <= 8 ? (size_t)B * C * 16 : (size_t)16 * (C + 1) * 16;
  if (x_bytes > GSA_MAX_X_LDS_BYTES) return false;
  ValuChoice k{nullptr, kMfmaWaves};
  switch (B) {
    case 1: k = valu_kernel<1>(C); break;
    case 2: k = valu_kernel<2>(C); break;
    case 3: k = valu_kernel<3>(C); break;
    case 4: k = valu_kernel<4>(C); break;
    case 5: k = valu_kernel<5>(C); break;
    case 6: k = valu_kernel<6>(C); break;
    case 7: k = valu_kernel<7>(C); break;
    case 8: k = valu_kernel<8>(C); break;
    default:
      k = {reinterpret_cast<const void*>(&gemv_ar_mfma<kMfmaWaves, 16, 1>), kMfmaWaves};
      break;
  }
  const unsigned block = (unsigned)(k.waves + 1) * 64;
  *out = {k.kernel, block, gemv_lds_bytes(W, B, C)};
  return true;
}

hipError_t launch_gemv(const Launch& l, const GemvArgs& a, hipStream_t s) {
  void* args[] = {const_cast<GemvArgs*>(&a)};
  return hipLaunchKernel(l.kernel, dim3((unsigned)a.tiles), dim3(l.block), args, l.lds_bytes, s);
}

hipError_t launch_pad_reset(uint32_t* pad, int W, int row_stride, int tiles,
                            uint32_t published_mask, hipStream_t s) {
  (void)tiles;
  const int64_t total = GSA_PAD_HEADER_WORDS + (int64_t)W * row_stride;
  const unsigned block = 256;
  const unsigned grid = (unsigned)((total + block - 1) / block);
  hipLaunchKernelGGL(pad_reset_kernel, dim3(grid), dim3(block), 0, s, pad, W, row_stride,
                     published_mask);
  return hipGetLastError();
}

}  // namespace gsa
