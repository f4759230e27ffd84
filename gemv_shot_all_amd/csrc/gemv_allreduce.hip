// gemv_allreduce.hip -- the fused GEMV + one-shot AllReduce kernels for gfx950.
//
// One workgroup owns one tile of TR output rows x all B batch columns: TR = 4
// (the plain one-shot call on short rows) or 16 (everything else).  The
// signal pad holds one flag per rank per flag tile of 4 rows, so a workgroup
// raises and waits on TR / 4 flags.  Inside one launch it
//   a. reads its own flags (epoch e = flag + 1 per flag tile) and polls the
//      peers' flags for its rows; if every peer has already published (always
//      the case for simulated peers) it acquires and prefetches the peer slots
//      so their latency hides under the A stream;
//   b. stages this rank's activation slice x (bf16) in LDS;
//   c. streams its 16 rows of A_r with 128-bit loads and multiply-adds in
//      fp32 (VALU bf16 dot2 for B <= 8, MFMA 16x16x32 for 8 < B <= 16);
//   d. reduces lane partials with a fixed DPP / lane-swap tree (or, for MFMA, a fixed
//      cross-wave sum through LDS);
//   e. publishes y into slot[rank], releases flag[rank][f] = e for each of
//      its flag tiles f, waits (if step a did not already see them) for every
//      peer's flag >= e, and writes out = ((0 + s_0) + s_1) ... + s_{W-1} in
//      rank order (rows of a flag tile whose wait expired stay unwritten).
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
//
// Memory ordering of the signal-pad protocol.  Every access to shared
// protocol state -- the published slot values, the peer slot values and the
// flags -- is an agent-scope atomic (relaxed), which gfx950 performs at the
// device coherence point, past the per-XCD L2 (sc1 loads and stores).  The
// writer makes its slot stores complete (s_waitcnt vmcnt(0)) before the
// workgroup barrier that precedes the flag store; the reader issues its slot
// loads only after the flag load has returned a value >= the epoch (the loads
// sit behind a branch on that value).  That orders data before flag without
// an agent-scope fence, whose whole-L2 writeback (release) or invalidate
// (acquire) per workgroup would cost several microseconds per call.  Across
// GPUs the same scheme runs at system scope.

#include <algorithm>
#include <type_traits>

#include "gsa_device.h"
#include "gsa_internal.h"

namespace gsa {
namespace {

constexpr int kFlagRows = GSA_FLAG_TILE_ROWS;  // rows per flag tile (4)
constexpr int kBigTile = 16;                   // rows of the MFMA / epilogue / two-shot tiles
constexpr int kMaxW = GSA_MAX_W;
static_assert(kBigTile % kFlagRows == 0 && kBigTile / kFlagRows * kMaxW <= 64,
              "one communication-wave lane per (flag tile, rank) of a workgroup");

// Workgroup LDS control words:
//   s_ctl[0] after a late wait: bit q set if flag tile q of the workgroup is complete
//   s_ctl[1] what the start-of-kernel poll found (kMustWait / kPeersReady /
//            kBadOwnRow), after a late wait kPeersReady if every flag tile is complete
//   s_ctl[2], s_ctl[3] the fused epilogue's (see fused_epilogue)
//   s_ctl[4 + q] the epoch of flag tile q
//   s_ctl[8] 0 from B1 (the VALU compute waves clear it before B1, so that no
//            LDS store delays B0), 1 once the communication wave has stored
//            the peer tile it loaded at the start (the compute waves may wait
//            for it without a barrier)
constexpr int kCtlWords = 9;
enum : uint32_t { kMustWait = 0u, kPeersReady = 1u, kBadOwnRow = 2u };

// The workgroup tile of this block.  The dispatcher deals consecutive block
// ids to the XCDs in turn (block b runs on XCD b % 8).  With XM the tiles go
// to the XCDs in contiguous runs instead, so the slot, out and flag lines of
// neighbouring tiles are written from one XCD (one L2); measured on the
// shorter rows, where those stores weigh most (8B down_proj shape 4.95
// against 5.08 us per call), and not taken on the longer rows or by MFMA
// (slightly slower there).
constexpr uint32_t kXcds = 8;
template <bool XM>
__device__ __forceinline__ int64_t block_tile() {
  const uint32_t b = blockIdx.x;
  if constexpr (!XM) {
    return b;
  } else {
    const uint32_t T = gridDim.x, x = b % kXcds, k = b / kXcds;
    const uint32_t per = T / kXcds, rem = T % kXcds;
    return (int64_t)(x * per + min(x, rem) + k);  // a bijection of [0, T)
  }
}

// The flag tiles [f0, f0 + nf) of workgroup tile `tile` of TR rows (the last
// workgroup may cover fewer than TR / 4 of the ceil(N / 4) flag tiles).
struct FlagSpan {
  int64_t f0;
  int nf;
};
template <int TR>
__device__ __forceinline__ FlagSpan flag_span(const GemvArgs& a, int64_t tile) {
  constexpr int FPW = TR / kFlagRows;
  const int64_t f0 = tile * FPW;
  const int64_t nflags = (a.N + kFlagRows - 1) / kFlagRows;
  return {f0, (int)min((int64_t)FPW, nflags - f0)};
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

// fp32 -> bf16 bits, round to nearest, ties to even; a NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Slot and output element types.  A buffer's slots hold fp32 or bf16 values
// (a.slot_bf16) and out is fp32 or bf16 (a.out_bf16); every sum is taken in
// fp32 either way.  Both flags are uniform over the launch, so each access
// below is one branch of a uniform condition.
//   publish_value: y as published into the own slot (its bf16 rounding for
//                  bf16 slots), which is also the own term of the rank-order
//                  sum, so that out is the fold of the slots as published;
//   load_slot:     element i of the slots (i = r * N * B + n * B + b),
//                  widened exactly to fp32; a device-coherent load;
//   load_slot_bits / slot_value: the same in two halves, for loads issued
//                  well before their use: one coherent 32-bit load with no
//                  branch (for bf16 slots the aligned word that holds
//                  element i; the slot region is padded to whole words), and
//                  the element's widening from that word.  A 16-bit load in
//                  a dtype branch has its zero-extension inside the branch,
//                  which waits for that load before the next one issues;
//   store_slot:    the device-coherent store of a published value;
//   store_out:     out[i], rounded to bf16 for a bf16 out (store_out_wt:
//                  the same, written through).
__device__ __forceinline__ float bf16_widen(uint16_t bits) {
  return __uint_as_float((uint32_t)bits << 16);
}
__device__ __forceinline__ float publish_value(const GemvArgs& a, float y) {
  return a.slot_bf16 ? bf16_widen(bf16_rne(y)) : y;
}
__device__ __forceinline__ uint32_t load_slot_bits(const GemvArgs& a, int64_t i) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t*>(a.slots) + (a.slot_bf16 ? i >> 1 : i),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float slot_value(const GemvArgs& a, int64_t i, uint32_t bits) {
  if (a.slot_bf16) bits = (i & 1) ? bits & 0xFFFF0000u : bits << 16;  // little-endian halves
  return __uint_as_float(bits);
}
__device__ __forceinline__ float load_slot(const GemvArgs& a, int64_t i) {
  return slot_value(a, i, load_slot_bits(a, i));
}
__device__ __forceinline__ void store_slot(const GemvArgs& a, int64_t i, float yp) {
  if (a.slot_bf16)
    __hip_atomic_store(reinterpret_cast<uint16_t*>(a.slots) + i,
                       (uint16_t)(__float_as_uint(yp) >> 16), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    store_coherent(a.slots + i, yp);
}
__device__ __forceinline__ void store_out(const GemvArgs& a, int64_t i, float o) {
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[i] = bf16_rne(o);
  else
    a.out[i] = o;
}
// out[i] written through to the coherence point like a published value,
// instead of left in L2 for the kernel's closing write-back; used by the
// publish path of the VALU and 16-row MFMA kernels (the small, o_proj and 8B
// down_proj shapes, fp32 or bf16 out: 0.05-0.16 us per call faster).  The
// long-row kernel measured no change with it and the LDS-staged MFMA kernel
// 0.45 us slower, so both keep store_out.
__device__ __forceinline__ void store_out_wt(const GemvArgs& a, int64_t i, float o) {
  if (a.out_bf16)
    __hip_atomic_store(reinterpret_cast<uint16_t*>(a.out) + i, bf16_rne(o), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    store_coherent(a.out + i, o);
}

// Element types of a kernel instance: fp32 slots and out, bf16 slots and
// out, or either (tested at run time).
constexpr int kDtF32 = 0;
constexpr int kDtMixed = 1;
constexpr int kDtBf16 = 2;

// The launch arguments as a kernel instance sees them: an fp32 or bf16
// instance fixes both element types, so every test of them above folds away
// at compile time (the run-time tests cost 0.2-0.4 us per call on the short
// rows, through the publish chain); calls with one of the two in bf16
// launch the mixed instance.
template <int DT>
__device__ __forceinline__ GemvArgs typed_args(const GemvArgs& args) {
  GemvArgs a = args;
  if constexpr (DT != kDtMixed) {
    a.slot_bf16 = DT == kDtBf16 ? 1 : 0;
    a.out_bf16 = DT == kDtBf16 ? 1 : 0;
  }
  return a;
}

// Word of flag tile t within a rank's row: groups of 4 flag tiles (one
// 16-row tile), one group per 128-byte line.
__device__ __forceinline__ int64_t flag_word(int64_t t) {
  return (t / GSA_FLAG_GROUP_TILES) * GSA_FLAG_GROUP_WORDS + t % GSA_FLAG_GROUP_TILES;
}
__device__ __forceinline__ uint32_t* flag_ptr(const GemvArgs& a, int r, int64_t t) {
  return a.pad + GSA_PAD_HEADER_WORDS + (int64_t)r * a.row_stride + flag_word(t);
}
// Two-shot: rank r's reduced-chunk flag for tile t (pad row W + r).
__device__ __forceinline__ uint32_t* flag2_ptr(const GemvArgs& a, int r, int64_t t) {
  return a.pad + GSA_PAD_HEADER_WORDS + (int64_t)(a.W + r) * a.row_stride + flag_word(t);
}
// The rank that reduces workgroup tile t of TR rows: the calling rank, or in
// the two-shot variant (TS) the owner of the tile's chunk (chunks are whole
// 16-row blocks, so a tile has one owner).  The kernels take TS as a template
// argument so that the one-shot instances carry none of this code.
template <bool TS, int TR>
__device__ __forceinline__ int tile_owner(const GemvArgs& a, int64_t t) {
  if constexpr (TS)
    return min(a.W - 1, (int)((uint32_t)t / (uint32_t)(a.chunk_tiles * (kBigTile / TR))));
  else
    return a.rank;
}

// The communication wave's flag lanes: lane l stands for rank p = l % 8 of
// the workgroup's flag tile q = l / 8 (lanes past the span, p >= W or
// q >= nf, are clamped to a valid word and ignored by the callers; no load
// sits under divergent control, and no division delays the first load).
__device__ __forceinline__ int lane_q(const FlagSpan& fs, int lane) {
  return min(lane >> 3, fs.nf - 1);
}
__device__ __forceinline__ bool lane_in_span(const GemvArgs& a, const FlagSpan& fs, int lane) {
  return (lane & 7) < a.W && (lane >> 3) < fs.nf;
}
__device__ __forceinline__ uint32_t load_flag(const GemvArgs& a, const FlagSpan& fs, int lane) {
  return __hip_atomic_load(flag_ptr(a, min(lane & 7, a.W - 1), fs.f0 + lane_q(fs, lane)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two-shot: lane q < nf reads the owner's reduced-chunk flag of flag tile q.
__device__ __forceinline__ uint32_t load_flag2(const GemvArgs& a, const FlagSpan& fs, int owner,
                                               int lane) {
  return __hip_atomic_load(flag2_ptr(a, owner, fs.f0 + min(lane, fs.nf - 1)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Peer tiles: rank r's TR x B tile of slot r lands at pe[(r * TR + n) * B + b]
// for every peer r != rank.  issue_peer_tile loads up to kPerLane values per
// lane per peer into registers, as raw bits (rows past N are clamped to a
// valid address; their values are never read); store_peer_tile widens them
// and writes them to LDS.  The peer loop is unrolled over GSA_MAX_W with a
// uniform guard, so no load sits under divergent control; nothing uses a
// loaded value inside its guard, so no load waits for the one before it.
template <int TR>
constexpr int kPerLane = (TR * GSA_MAX_B + 63) / 64;  // 4 (TR = 16) or 1 (TR = 4)

template <bool TS, int TR>
__device__ __forceinline__ void issue_peer_tile(const GemvArgs& a, int lane, int64_t tile,
                                                uint32_t (&v)[kMaxW][kPerLane<TR>]) {
  const int64_t NB = a.N * a.B;
  const int per_lane = (TR * a.B + 63) / 64;  // 1, 2 or 4
  const int64_t first = tile * TR * a.B;      // first element of the tile in a slot
  const int64_t last = NB - 1;
  const int owner = tile_owner<TS, TR>(a, tile);
  // Two-shot, a chunk another rank reduces: its published values, held in
  // v[0] (store_peer_tile puts them at the owner's place in the peer tile).
  const bool copy = TS && owner != a.rank;
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) {
    if (copy ? r == 0 : (r < a.W && r != a.rank)) {
#pragma unroll
      for (int i = 0; i < kPerLane<TR>; ++i) {
        const int64_t e = min(first + lane + 64 * i, last);
        if (i < per_lane)
          v[r][i] = copy ? __float_as_uint(load_coherent(&a.gathered[e]))
                         : load_slot_bits(a, r * NB + e);
      }
    }
  }
}

template <bool TS, int TR>
__device__ __forceinline__ void store_peer_tile(const GemvArgs& a, int lane, int64_t tile,
                                                const uint32_t (&v)[kMaxW][kPerLane<TR>],
                                                float* pe) {
  const int64_t NB = a.N * a.B;
  const int tb = TR * a.B;  // elements of one rank's tile
  const int per_lane = (tb + 63) / 64;
  const int64_t first = tile * tb;
  const int owner = tile_owner<TS, TR>(a, tile);
  const bool copy = TS && owner != a.rank;  // v[0] holds the owner's values
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) {
    if (copy ? r == 0 : (r < a.W && r != a.rank)) {
      float* dst = pe + (copy ? owner : r) * tb;
#pragma unroll
      for (int i = 0; i < kPerLane<TR>; ++i) {
        const int e = lane + 64 * i;
        const int64_t g = min(first + e, NB - 1);  // the element issue_peer_tile loaded
        if (i < per_lane && e < tb)
          dst[e] = copy ? __uint_as_float(v[r][i]) : slot_value(a, r * NB + g, v[r][i]);
      }
    }
  }
}

// The communication wave's start: derive each flag tile's epoch from its own
// flag and check every peer's flag for it.  Writes s_ctl[4 + q] = epoch of
// flag tile q and s_ctl[1] = kMustWait / kPeersReady / kBadOwnRow; returns
// s_ctl[1].  A workgroup with an unusable own flag (marked published, or its
// epochs exhausted) records the first such flag tile and does nothing else.
template <bool TS, int TR>
__device__ __forceinline__ uint32_t comm_decide(const GemvArgs& a, int lane, int64_t tile,
                                                const FlagSpan& fs, uint32_t fl, uint32_t* s_ctl) {
  const int q = lane_q(fs, lane);
  const int p = lane & 7;
  const bool in_span = lane_in_span(a, fs, lane);
  const uint32_t own = __shfl(fl, q * 8 + a.rank);  // the own flag of this lane's flag tile
  const uint64_t bad = __ballot(in_span && own >= GSA_FLAG_PUBLISHED - 1u);
  if (bad != 0) {
    if (lane == 0) {
      atomicOr(a.pad + kHdrErrorBits, kErrState);
      atomicMin(a.pad + kHdrStateTile,
                (uint32_t)(fs.f0 + ((__ffsll((long long)bad) - 1) >> 3)));
      s_ctl[1] = kBadOwnRow;
    }
    return kBadOwnRow;
  }
  const uint32_t epoch = own + 1u;
  if (in_span && p == a.rank) s_ctl[4 + q] = epoch;
  const int owner = tile_owner<TS, TR>(a, tile);
  bool lane_ok = !in_span || p == a.rank || fl >= epoch;
  if (TS && owner != a.rank) {  // two-shot: only the owner's reduced chunk is needed
    const uint32_t e2 = __shfl(fl, min(lane, fs.nf - 1) * 8 + a.rank) + 1u;
    const uint32_t f2 = load_flag2(a, fs, owner, lane);  // every lane loads a valid word
    lane_ok = lane >= fs.nf || f2 >= e2;
  }
  const bool ready = __ballot(!lane_ok) == 0;
  if (lane == 0) s_ctl[1] = ready ? kPeersReady : kMustWait;
  return ready ? kPeersReady : kMustWait;
}

// Bounded wait for every peer's flag >= the epoch of each of the workgroup's
// flag tiles.  Returns the mask of complete flag tiles (bit q); on expiry
// records the smallest missing (flag tile, peer) in the pad header.
template <bool TS, int TR>
__device__ uint32_t wait_peers(const GemvArgs& a, int lane, int64_t tile, const FlagSpan& fs,
                               const uint32_t* s_ctl) {
  const uint64_t start = wall_clock64();
  const int owner = tile_owner<TS, TR>(a, tile);
  const bool copy = TS && owner != a.rank;  // two-shot: the owner's reduced-chunk flags
  const int q = copy ? min(lane, fs.nf - 1) : lane_q(fs, lane);
  const bool in_span = copy ? lane < fs.nf : lane_in_span(a, fs, lane);
  const int p = lane & 7;
  const uint32_t epoch = s_ctl[4 + q];
  const uint32_t all = (1u << fs.nf) - 1u;
  for (;;) {
    // Every lane loads a valid word; lanes outside the span are ignored.
    const uint32_t f = copy ? load_flag2(a, fs, owner, lane) : load_flag(a, fs, lane);
    const bool lane_ok = !in_span || (!copy && p == a.rank) || f >= epoch;
    const uint64_t missing = __ballot(!lane_ok);
    if (missing == 0) return all;
    if (wall_clock64() - start > a.timeout_ticks) {
      uint32_t failed = 0;
      for (int f = 0; f < fs.nf; ++f) {
        const uint64_t lanes = copy ? (1ull << f) : (0xFFull << (8 * f));
        if (missing & lanes) failed |= 1u << f;
      }
      if (lane == 0) {
        const int l = __ffsll((long long)missing) - 1;
        const int64_t f = fs.f0 + (copy ? l : l >> 3);
        const uint32_t peer = copy ? (uint32_t)owner : (uint32_t)(l & 7);
        atomicOr(a.pad + kHdrErrorBits, kErrTimeout);
        atomicMin(a.pad + kHdrTimeoutKey, (uint32_t)f * 8u + peer);
      }
      return all & ~failed;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The fused epilogue's grouped counts (see kEpiGroups): 16-row tile t is in
// group t % kEpiGroups, which holds epi_group_tiles(g) of the call's 16-row
// tiles (a workgroup of more rows counts each of its 16-row tiles).
__device__ __forceinline__ int epi_group_tiles(const GemvArgs& a, int g) {
  return g < a.epi_tiles ? (a.epi_tiles - g + kEpiGroups - 1) / kEpiGroups : 0;
}

__device__ __forceinline__ unsigned long long* epi_count(const GemvArgs& a, int64_t off, int g) {
  return reinterpret_cast<unsigned long long*>(a.ssq + off + (int64_t)g * kEpiRecordWords);
}

// Count 16-row tile t16 started (lanes below `subs` count t16 + lane, if it
// exists); returns the count lane 0 saw before its own (used only in lane 0).
__device__ __forceinline__ unsigned long long epi_count_started(const GemvArgs& a, int64_t t16,
                                                                int subs, int lane) {
  unsigned long long before = 0;
  if (lane < subs && t16 + lane < a.epi_tiles)
    before = __hip_atomic_fetch_add(
        epi_count(a, epi_started_off(a.epi_tiles), (int)((t16 + lane) % kEpiGroups)), 1ull,
        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return before;
}

// Lane g's reading of group g's started count (0 for a group without tiles).
__device__ __forceinline__ unsigned long long epi_started_load(const GemvArgs& a, int lane) {
  return epi_group_tiles(a, lane) > 0
             ? __hip_atomic_load(epi_count(a, epi_started_off(a.epi_tiles), lane),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
             : 0ull;
}

// Once the workgroup's protocol work is done: the call's index k (from the
// count lane 0 saw for 16-row tile t16, every tile of a call being counted
// once in its group) into *s_epi_k, and into s_ctl[3] whether every 16-row
// tile of the call had started when the counts `now` (epi_started_load, lane
// g: group g) were read.  One wave.
__device__ __forceinline__ void epi_note_started(const GemvArgs& a, int64_t t16,
                                                 unsigned long long before,
                                                 unsigned long long now, int lane,
                                                 uint32_t* s_ctl, unsigned long long* s_epi_k) {
  const int grp = (int)(t16 % kEpiGroups);
  const unsigned long long k =
      __builtin_amdgcn_readfirstlane((uint32_t)(before / (unsigned)epi_group_tiles(a, grp))) |
      0ull;
  const int ng = epi_group_tiles(a, lane);
  const bool lane_ok = ng == 0 || now >= (k + 1ull) * (unsigned)ng;
  const bool all_started = __ballot(!lane_ok) == 0;
  if (lane == 0) {
    *s_epi_k = k;
    s_ctl[3] = all_started ? 1u : 0u;
  }
}

// The kernels' epilogue parameter EPI: none, the fused bias + RMSNorm with
// 1/rms folded by one workgroup and polled by the others, or folded by every
// workgroup that waits (few records: no copy of 1/rms to publish and poll).
constexpr int kEpiNone = 0, kEpiFoldOne = 1, kEpiFoldAll = 2;
constexpr int64_t kEpiFoldAllWords = 64;  // kEpiFoldAll up to this many record words a call

// The workgroup of tile `tile` (TR rows) folds the epilogue's records if it
// holds the call's last 16-row tile.
template <int TR>
__device__ __forceinline__ bool epi_reducer(const GemvArgs& a, int64_t tile) {
  static_assert(TR % kBigTile == 0, "whole 16-row tiles");
  return (a.epi_tiles - 1) / (TR / kBigTile) == tile;
}

// The communication wave (the last wave of every workgroup) runs the
// signal-pad protocol, so its round trips never hold up the A stream of the
// compute waves.  A CU returns vector loads in issue order, so the flag load
// goes out before the compute waves' x and A loads (barrier B0); the peer
// loads it issues once the flags are back return right behind the A stream.
// Barrier schedule shared with the compute waves:
//   B0 flag load issued | B1 decision in s_ctl (the VALU kernels: x staged;
//   the MFMA kernels: per-wave partials in LDS) | B2 own slot published, and
//   the peer tile in LDS if the peers were ready at the start (lanes of
//   compute wave 0 then store the workgroup's flags) | B3 (only if they were
//   not) late peer tile in LDS | two-shot, own chunk: B5 (reduced chunk
//   published; compute wave 0 then stores the reduced-chunk flags) | with the
//   fused epilogue: E1, E2 and
//   maybe E3, E4 (see fused_epilogue).
// The peer loads stay in flight across B1: a workgroup barrier does not wait
// for outstanding global loads.
// With the epilogue the communication wave also counts the tile started in
// its group (after B0) and, once its protocol work is done, looks whether
// every tile of the call has started (s_ctl[3]: lane g reads group g's
// count); s_epi_k gets the call's index.
// PE: whether the compute waves take the peer tile from LDS when every peer
// had published at the start (the VALU one-shot kernels load their own peer
// values instead; a late peer tile always goes through LDS).
template <bool TS, int TR, bool PE, int EPI>
__device__ void comm_wave(const GemvArgs& a, int lane, int64_t tile, float* pe,
                          uint32_t* s_ctl, unsigned long long* s_epi_k) {
  const FlagSpan fs = flag_span<TR>(a, tile);
  const uint32_t fl = load_flag(a, fs, lane);
  __syncthreads();  // B0: the flag loads are issued ahead of every x and A load
  // Count the tile started; the value is used only after the protocol work.
  constexpr bool kEpi = EPI != 0 && TR == kBigTile;  // the epilogue runs on 16-row tiles here
  unsigned long long before = 0;
  if constexpr (kEpi) before = epi_count_started(a, tile, 1, lane);
  const uint32_t state = comm_decide<TS, TR>(a, lane, tile, fs, fl, s_ctl);
  uint32_t v[kMaxW][kPerLane<TR>];
  const bool early_tile = PE && state == kPeersReady;
  if (early_tile) issue_peer_tile<TS, TR>(a, lane, tile, v);  // after the flags returned
  __syncthreads();  // B1
  if (early_tile) {
    store_peer_tile<TS, TR>(a, lane, tile, v, pe);
    // The mark is a workgroup-scope release: every lane's peer-tile stores
    // above happen before it, for the compiler and for the hardware alike
    // (its acquire load is in the compute waves).
    if (lane == 0)
      __hip_atomic_store(&s_ctl[8], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();  // B2
  if (state == kMustWait) {
    // The own flags went out after B2.
    const uint32_t done = wait_peers<TS, TR>(a, lane, tile, fs, s_ctl);
    if (done != 0) {
      // After the flags returned; rows of incomplete flag tiles are never read.
      issue_peer_tile<TS, TR>(a, lane, tile, v);
      store_peer_tile<TS, TR>(a, lane, tile, v, pe);
    }
    if (lane == 0) {
      s_ctl[0] = done;
      s_ctl[1] = done == (1u << fs.nf) - 1u ? kPeersReady : kMustWait;
    }
    __syncthreads();  // B3
  }
  if (TS && tile_owner<TS, TR>(a, tile) == a.rank) __syncthreads();  // B5
  if constexpr (kEpi) {
    epi_note_started(a, tile, before, epi_started_load(a, lane), lane, s_ctl, s_epi_k);
    __syncthreads();  // E1
    __syncthreads();  // E1b
    if (s_ctl[3] || epi_reducer<TR>(a, tile)) {  // a waiting tile, or the reducing workgroup
      __syncthreads();  // E3
      __syncthreads();  // E4
    }
  }
}

// out = ((0 + s_0) + s_1) ... + s_{W-1}; s_rank is this call's published y,
// the others come from the peer tile in LDS (local row n, column b).  The W
// peer values are read up front (indexes clamped into the tile) and ranks
// r >= W add +0: the sum starts at +0 and a round-to-nearest sum is -0 only
// if both terms are, so acc is never -0 and acc + 0 == acc exactly.
template <int TR>
__device__ __forceinline__ float one_shot_sum(const GemvArgs& a, float y, const float* pe, int n,
                                              int b) {
  const int tb = TR * a.B;
  const int idx = n * a.B + b;
  float pv[kMaxW];
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) pv[r] = pe[min(r, a.W - 1) * tb + idx];
  float acc = 0.0f;
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) {
    const float t = r == a.rank ? y : pv[r];
    acc = acc + (r < a.W ? t : 0.0f);
  }
  return acc;
}

template <int BM, int OPL, int TR, bool ALL>
__device__ void fused_epilogue(const GemvArgs& a, int64_t tile, const int (&n)[OPL], int b,
                               const bool (&own)[OPL], const bool (&live)[OPL],
                               const float (&o)[OPL], const bool (&ok)[OPL], float* elds,
                               uint32_t* s_ctl, const unsigned long long* s_epi_k, int wave,
                               int lane, int nt);

// Compute waves once y is final (y[e] for local row n[e], column b, if own[e]:
// every (row, column) of the tile has exactly one owner lane), `state` being
// what the communication wave decided before B1: publish y into slot[rank],
// B2, lanes of compute wave 0 release the workgroup's flags, [B3], out (rows
// of complete flag tiles), [the fused epilogue].  Every compute wave waits
// for its own slot stores to complete before B2, so the flag stores that
// follow B2 are ordered after all of them.  nt: compute threads of the
// workgroup.
//
// own_peers (the VALU one-shot kernels, every peer published at the start):
// the lane already holds its output's peer values in pv (loaded after B1),
// so out is summed and stored right behind the published value, and the
// wait before B2 covers only the published value (stores complete in issue
// order); the out store's round trip overlaps it.
template <int BM, int OPL, bool TS, int TR, int EPI>
__device__ __forceinline__ void publish_and_reduce(const GemvArgs& a, int64_t tile, const int (&n)[OPL], int b,
                                   const bool (&own)[OPL], const float (&y)[OPL],
                                   const float* pe, float* elds, uint32_t* s_ctl,
                                   const unsigned long long* s_epi_k, uint32_t state, int wave,
                                   int lane, int nt, bool own_peers,
                                   const float (&pv)[kMaxW]) {
  static_assert(OPL == 1, "one output per lane");
  const int64_t NB = a.N * a.B;
  const int64_t row0 = tile * TR;
  const FlagSpan fs = flag_span<TR>(a, tile);
  bool live[OPL];
  float yp[OPL];  // y as published (the own term of the sum)
#pragma unroll
  for (int e = 0; e < OPL; ++e) {
    live[e] = own[e] && row0 + n[e] < a.N;
    yp[e] = publish_value(a, y[e]);
  }
  float o[OPL];
  bool ok[OPL];
  if (own_peers) {
    // out = ((0 + s_0) + s_1) ... + s_{W-1}, the own term being y as
    // published; the same order and operations as one_shot_sum.  Summed
    // before the published value is stored, so that waiting for the peer
    // values cannot wait for that store.
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < kMaxW; ++r) {
      const float t = r == a.rank ? yp[0] : pv[r];
      acc = acc + (r < a.W ? t : 0.0f);
    }
    o[0] = acc;
    ok[0] = true;
  }
  // Nothing may move across: the waits below count on every load being
  // complete here and on the published value being issued before the out
  // store.
  __builtin_amdgcn_sched_barrier(0);
  if (state != kBadOwnRow) {
#pragma unroll
    for (int e = 0; e < OPL; ++e)
      if (live[e]) store_slot(a, a.rank * NB + (row0 + n[e]) * a.B + b, yp[e]);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (own_peers) {
    if (live[0]) {
      const int64_t i = (row0 + n[0]) * a.B + b;
      if constexpr (EPI)
        store_coherent(&a.out[i], o[0]);  // the reducing workgroup may read it back
      else
        store_out_wt(a, i, o[0]);
    }
    wait_vm_le<1>();  // the published value is at the coherence point ...
  } else {
    wait_vm_all();    // the published values are at the coherence point ...
  }
  __syncthreads();  // B2 ... in every compute wave
  if (state != kBadOwnRow && wave == 0 && lane < fs.nf)
    store_flag(flag_ptr(a, a.rank, fs.f0 + lane), s_ctl[4 + lane]);
  uint32_t done = state == kBadOwnRow ? 0u : ~0u;  // complete flag tiles
  if (state == kMustWait) {
    __syncthreads();  // B3
    done = s_ctl[0];  // a wait expired: those flag tiles' out rows stay unwritten
  }
  const int owner = tile_owner<TS, TR>(a, tile);
#pragma unroll
  for (int e = 0; e < OPL; ++e) {
    if (own_peers) break;  // out already stored
    ok[e] = ((done >> (n[e] / kFlagRows)) & 1u) != 0;
    o[e] = 0.0f;
    if (ok[e] && live[e]) {
      const int64_t i = (row0 + n[e]) * a.B + b;
      if (!TS || owner == a.rank) {
        o[e] = one_shot_sum<TR>(a, yp[e], pe, n[e], b);
        if (TS) store_coherent(&a.gathered[i], o[e]);  // this rank's reduced chunk
      } else {
        o[e] = pe[owner * TR * a.B + n[e] * a.B + b];  // the owner's reduced chunk
      }
      if constexpr (EPI)
        store_coherent(&a.out[i], o[e]);  // the reducing workgroup may read it back
      else
        store_out_wt(a, i, o[e]);
    }
  }
  if (TS && owner == a.rank) {
    wait_vm_all();    // the reduced chunk is at the coherence point ...
    __syncthreads();  // B5 ... in every compute wave
    if (wave == 0 && lane < fs.nf && ((done >> lane) & 1u))
      store_flag(flag2_ptr(a, a.rank, fs.f0 + lane), s_ctl[4 + lane]);
  }
  if constexpr (EPI != kEpiNone && TR == kBigTile)
    fused_epilogue<BM, OPL, TR, EPI == kEpiFoldAll>(a, tile, n, b, own, live, o, ok, elds, s_ctl,
                                                    s_epi_k, wave, lane, nt);
}

// The value that lane l ^ D holds (D = 8, 4, 2 or 1; partners stay within a
// 16-lane row).  D = 8 and 4 take two DPP row shifts, each writing only the
// 4-lane banks whose partner lies in its direction; D = 2 and 1 one quad
// permutation.
template <int D>
__device__ __forceinline__ float partner_value(float v) {
  auto dpp = [](float old, float src, auto ctrl, auto bank) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                           __builtin_bit_cast(int, src), decltype(ctrl)::value,
                                           0xF, decltype(bank)::value, false));
  };
  using I = int;
  if constexpr (D == 8) {
    const float t = dpp(0.0f, v, std::integral_constant<I, 0x108>{},   // row_shl:8
                        std::integral_constant<I, 0x3>{});             // banks 0, 1
    return dpp(t, v, std::integral_constant<I, 0x118>{},               // row_shr:8
               std::integral_constant<I, 0xC>{});                      // banks 2, 3
  } else if constexpr (D == 4) {
    const float t = dpp(0.0f, v, std::integral_constant<I, 0x104>{},   // row_shl:4
                        std::integral_constant<I, 0x5>{});             // banks 0, 2
    return dpp(t, v, std::integral_constant<I, 0x114>{},               // row_shr:4
               std::integral_constant<I, 0xA>{});                      // banks 1, 3
  } else if constexpr (D == 2) {
    return dpp(0.0f, v, std::integral_constant<I, 0x4E>{},             // quad_perm [2,3,0,1]
               std::integral_constant<I, 0xF>{});
  } else {
    static_assert(D == 1, "partner distance 8, 4, 2 or 1");
    return dpp(0.0f, v, std::integral_constant<I, 0xB1>{},             // quad_perm [1,0,3,2]
               std::integral_constant<I, 0xF>{});
  }
}

// One stage of a reduce-scatter at lane distance D over V values per lane:
// lane l keeps the upper half of the values if bit D of l is set, else the
// lower half, and adds the partner's copy of the half it keeps.  V == 1: a
// plain pairwise sum (both lanes end with the same total).
template <int D, int V, int N>
__device__ __forceinline__ void rs_stage(float (&v)[N], int lane) {
  static_assert(V <= N, "stage over the array's first V values");
  if constexpr (V == 1) {
    if constexpr (D >= 16) {
      const unsigned u = __builtin_bit_cast(unsigned, v[0]);
      const auto p = D == 32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane16_swap(u, u, false, false);
      v[0] = __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
    } else {
      v[0] = v[0] + partner_value<D>(v[0]);
    }
  } else if constexpr (D >= 16) {
    // The swap pairs rows (16 or 32 lanes) so that each lane ends with its own
    // and its partner's copy of the half it keeps.
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      const unsigned lo = __builtin_bit_cast(unsigned, v[j]);
      const unsigned hi = __builtin_bit_cast(unsigned, v[j + V / 2]);
      const auto p = D == 32 ? __builtin_amdgcn_permlane32_swap(lo, hi, false, false)
                             : __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
      v[j] = __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
    }
  } else {
    const bool upper = (lane & D) != 0;
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      const float keep = upper ? v[j + V / 2] : v[j];
      const float give = upper ? v[j] : v[j + V / 2];
      v[j] = keep + partner_value<D>(give);
    }
  }
}

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }
constexpr int log2_exact(int v) { return v <= 1 ? 0 : 1 + log2_exact(v / 2); }

// Reduce-scatter over the 64 lanes of a wave: v[0..V) are every lane's
// partials of V outputs (V a power of two, at most 64); afterwards v[0] of
// lane l holds the total over all 64 lanes of output l >> (6 - log2 V), in
// every lane of that output's aligned group of 64 / V lanes.  A fixed tree
// (bit-identical in every lane of a group, and from call to call).
template <int V>
__device__ __forceinline__ float reduce_scatter64(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "a power of two up to 64");
  rs_stage<32, (V >= 2 ? V : 1)>(v, lane);
  rs_stage<16, (V >= 4 ? V / 2 : 1)>(v, lane);
  rs_stage<8, (V >= 8 ? V / 4 : 1)>(v, lane);
  rs_stage<4, (V >= 16 ? V / 8 : 1)>(v, lane);
  rs_stage<2, (V >= 32 ? V / 16 : 1)>(v, lane);
  rs_stage<1, (V >= 64 ? V / 32 : 1)>(v, lane);
  return v[0];
}

// The same over each aligned group of 32 lanes (the two halves of a wave
// reduce separately): afterwards v[0] of lane l holds the total over its
// group of output (l & 31) >> (5 - log2 V), in every lane of that output's
// aligned group of 32 / V lanes.
template <int V>
__device__ __forceinline__ float reduce_scatter32(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 32 && (V & (V - 1)) == 0, "a power of two up to 32");
  rs_stage<16, (V >= 2 ? V : 1)>(v, lane);
  rs_stage<8, (V >= 4 ? V / 2 : 1)>(v, lane);
  rs_stage<4, (V >= 8 ? V / 4 : 1)>(v, lane);
  rs_stage<2, (V >= 16 ? V / 8 : 1)>(v, lane);
  rs_stage<1, (V >= 32 ? V / 16 : 1)>(v, lane);
  return v[0];
}

// The call's mark in the epilogue's scratch: 1 + k mod (2^31 - 1) for call
// index k, never 0 (cleared scratch reads 0) and below 2^31, so that the top
// bit of a record's tag can say that the tile left its rows to the reducing
// workgroup (kEpiLeft).
constexpr uint32_t kEpiLeft = 0x80000000u;
__device__ __forceinline__ uint32_t epi_mark(unsigned long long k) {
  return (uint32_t)(k % 0x7FFFFFFFull) + 1u;
}
__device__ __forceinline__ unsigned long long* epi_record(const GemvArgs& a, int64_t t) {
  return reinterpret_cast<unsigned long long*>(a.ssq + t * kEpiRecordWords);
}

// Sum of v over the lanes of the wave whose index agrees with this lane's
// modulo 2^lp (0 <= lp <= 5, wave-uniform, every lane active): a fixed
// butterfly at lane distances 2^lp, ..., 32 (DPP within 16-lane rows, then
// the two permlane swaps); every lane of a class ends with the same bits.
__device__ __forceinline__ float sum_lane_class(float v, int lp) {
  if (lp <= 0) v = v + partner_value<1>(v);
  if (lp <= 1) v = v + partner_value<2>(v);
  if (lp <= 2) v = v + partner_value<4>(v);
  if (lp <= 3) v = v + partner_value<8>(v);
  if (lp <= 4) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
  }
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

// 1 / rms per column, folded by the reducing workgroup from every tile's
// record as the records arrive.  Record t holds B 64-bit words; word c is
// (tag << 32) | the fp32 bits of tile t's sum of squares of column c, with
// tag = the call's mark, plus kEpiLeft if the tile left its rows.  A word is
// written and read whole, so it carries its own validity: no flag and no
// wait stand between a tile's sums and the fold.  P = B rounded up to a
// power of two lanes read one record (lane class c = lane mod P: column c);
// thread group j = (wave * 64 + lane) / P takes tiles j, j + nt / P, ... in
// ascending order, kLoads tiles' loads in flight, and re-reads the words that
// do not show this call's mark yet, together, until all do (bounded: twice
// the wait timeout).  The lanes of
// a class are summed by a fixed butterfly (sum_lane_class) and the waves'
// sums in wave order, so the result has the same bits on every call.
// Result in s_inv[0..B), NaN in every column if the wait expired (then the
// pad header records kErrEpiWait with flag tile ft0, the workgroup's first).
// s_ctl[2] must be 0 on entry.  Contains the barrier E3.
__device__ void fold_records(const GemvArgs& a, uint32_t mark, int64_t ft0, int wave, int lane,
                             int nt, float* wsum, float* s_inv, uint32_t* s_ctl,
                             bool prewait_wide) {
  constexpr int kLoads = 16;
  const int lp = a.B <= 1 ? 0 : 32 - __builtin_clz((unsigned)(a.B - 1));  // log2 P
  const int c = lane & ((1 << lp) - 1);
  const int groups = nt >> lp;
  const uint64_t limit = 2 * a.timeout_ticks + 1000000ull;
  const uint64_t start = wall_clock64();
  float acc = 0.0f;
  bool expired = false;
  if (lp > 0 && (lp <= 3 || prewait_wide)) {
    // 2 <= B <= 8 (B > 8 too if prewait_wide): first the column-0 word of
    // every record this wave reads below, the P lanes of a thread group
    // sharing its tiles.  A record's words are stored by one instruction, so
    // once these show the mark the reads below rarely find a word without
    // it, each of which would cost a round trip of its own there (8B
    // down_proj shape, B = 8: 11.1 against 12.2 us per call).  At B = 16 (32
    // words a lane) it pays only where the folding workgroup tends to finish
    // its own rows early, among others that run alongside it (the 32-row
    // LDS-staged kernel: skinny GEMM 15.7 against 18.1 us; the 16-row MFMA
    // kernel, whose last workgroup starts last: 18.0 against 16.6).
    const int j = (wave * 64 + lane) >> lp;
    for (int t = j + c * groups; t < a.epi_tiles && !expired; t += groups << lp) {
      unsigned long long v =
          __hip_atomic_load(epi_record(a, t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while (((uint32_t)(v >> 32) & ~kEpiLeft) != mark) {
        if (wall_clock64() - start > limit) {
          expired = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(epi_record(a, t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (c < a.B) {
    for (int t0 = (wave * 64 + lane) >> lp; t0 < a.epi_tiles; t0 += kLoads * groups) {
      unsigned long long w[kLoads];
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int t = min(t0 + u * groups, a.epi_tiles - 1);
        w[u] = __hip_atomic_load(epi_record(a, t) + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int t = t0 + u * groups;
        if (t < a.epi_tiles) {
          unsigned long long v = w[u];
          while (((uint32_t)(v >> 32) & ~kEpiLeft) != mark && !expired) {
            if (wall_clock64() - start > limit) {
              expired = true;
            } else {
              __builtin_amdgcn_s_sleep(1);
              v = __hip_atomic_load(epi_record(a, t) + c, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          acc = acc + (expired ? __builtin_nanf("") : __uint_as_float((uint32_t)v));
        }
      }
    }
  }
  acc = sum_lane_class(acc, lp);
  if (lane < (1 << lp)) wsum[wave * 16 + lane] = acc;
  if (__ballot(expired) != 0 && lane == 0) s_ctl[2] = 1u;
  __syncthreads();  // E3: every wave's sums in LDS
  if (wave == 0) {
    const bool failed = s_ctl[2] != 0;
    if (failed && lane == 0) {
      atomicOr(a.pad + kHdrErrorBits, kErrEpiWait);
      atomicMin(a.pad + kHdrEpiWaitTile, (uint32_t)ft0);
    }
    if (lane < a.B) {
      float tot = 0.0f;
      for (int w = 0; w < nt / 64; ++w) tot = tot + wsum[w * 16 + lane];
      s_inv[lane] = failed ? __builtin_nanf("") : 1.0f / sqrtf(tot / (float)a.N + a.eps);
    }
  }
}

__device__ __forceinline__ void store_y(const GemvArgs& a, int64_t i, float v) {
  if (a.y_bf16)
    static_cast<uint16_t*>(a.y)[i] = bf16_rne(v);
  else
    static_cast<float*>(a.y)[i] = v;
}

// The fused epilogue: bias, then RMSNorm over the N rows of every token
// column, then y in fp32 or bf16 ("PyTorch Symmetric Memory" talk, real-model
// example: the bias addition joins the reduction loop and the RMSNorm runs in
// the same kernel; RMSNorm by its textbook definition; bf16 output of an fp32
// accumulation as in the documentation's higher-precision reduction).
//   z = out + bias[n]; inv[b] = 1 / sqrtf(sum_n z^2 / N + eps);
//   y = (z * inv[b]) * w[n]
// The sum over n crosses workgroups.  Each tile sums its 16 squares per
// column in row order and publishes them as its record (fold_records: one
// self-validating 64-bit word per column, tagged with the call's mark).  The
// reducing workgroup, the last tile's (dispatched last, so most records are
// out when it starts reading them), folds every record as it arrives and
// publishes inv in kEpiGroups copies, one per group of tiles (t %
// kEpiGroups), as one 64-bit word per column holding the mark and the bits
// of inv.  No count stands between a record and the fold: against the
// earlier scheme (each tile counting itself done in its group, the tile that
// completed the count of groups folding), one wait for the records'
// acknowledgement and two atomic round trips fewer (us per call: c1 8.6 ->
// 7.5, o_proj 8.6 -> 7.8, 8B down_proj B = 1 9.9 -> 9.1, B = 4 10.2 -> 9.9;
// B = 8, the 70B-class shape and the skinny GEMM within their run-to-run
// spread).  The call index k comes from the started
// counts, which only grow (taken by the communication wave at entry), so no
// host state is needed (graph replays work).
//  - A tile that saw every tile of its call started (s_ctl[3], looked up by
//    the communication wave) may wait: every other tile is resident or done
//    and finishes on its own.  It polls (bounded) its group's copy until
//    every column shows the mark, takes inv from it and normalises its own
//    rows from registers.  With ALL (calls of at most 64 record words) it
//    folds the records itself instead, as the reducing workgroup does and
//    with the same bits, and no copy of inv is published: one store and one
//    poll fewer after the last record (c1 shape: 6.9 against 7.4 us per call
//    with one folding workgroup); from 256 tiles on, every tile reading
//    every record costs more than it saves (o_proj shape 8.0 against 7.8,
//    70B-class shape 21.3 against 16.8).
//  - Any other tile first waits until its out stores are at the coherence
//    point, tags its record kEpiLeft and leaves; the reducing workgroup, once
//    it has inv, also normalises the rows of every tile tagged so, re-reading
//    out (stored coherently for this).
// The reducing workgroup waits whatever it saw at its start: it holds one
// workgroup's place, and every tile it waits for has started or will start
// in a place that tiles leaving free up.  A row that failed (its flag tile's
// wait expired, or a bad own row) contributes NaN, so y comes out NaN for
// that call.  Barriers: E1 (squares in LDS), E1b (out stores complete in a
// tile that leaves), then, in the reducing and the waiting tiles, E3 (wave
// sums in LDS, or inv seen) and E4 (inv in LDS).
// The records, the counts and the copies of inv are kept per 16-row tile
// whatever the kernel's workgroup tile (TR = 16 or 32 rows, SUB = TR / 16
// records a workgroup), so that calls on one buffer through kernels of either
// tile size count and tag alike.  elds: TR x 16 squares, then 16 inv, then 8
// x 16 wave sums (floats).
template <int BM, int OPL, int TR, bool ALL>
__device__ void fused_epilogue(const GemvArgs& a, int64_t tile, const int (&n)[OPL], int b,
                               const bool (&own)[OPL], const bool (&live)[OPL],
                               const float (&o)[OPL], const bool (&ok)[OPL], float* elds,
                               uint32_t* s_ctl, const unsigned long long* s_epi_k, int wave,
                               int lane, int nt) {
  static_assert(TR % kBigTile == 0, "whole 16-row tiles");
  constexpr int SUB = TR / kBigTile;
  float* zz = elds;                 // [TR rows][16 columns] squares of z
  float* s_inv = elds + TR * 16;    // [16] 1 / rms per column
  float* wsum = s_inv + 16;         // [8 waves][16 columns] the fold's wave sums
  const int64_t row0 = tile * TR;
  const int64_t t16 = tile * SUB;   // the workgroup's first 16-row tile
  float z[OPL];
#pragma unroll
  for (int e = 0; e < OPL; ++e) {
    z[e] = 0.0f;
    if (own[e]) {
      float sq = 0.0f;  // rows past N add nothing
      if (live[e]) {
        z[e] = o[e] + (a.bias ? a.bias[row0 + n[e]] : 0.0f);
        sq = z[e] * z[e];
      }
      zz[n[e] * 16 + b] = ok[e] ? sq : __builtin_nanf("");
    }
  }
  __syncthreads();  // E1: the squares are in LDS
  const uint32_t mark = epi_mark(*s_epi_k);
  const bool waits = s_ctl[3] != 0;
  const bool reducer = epi_reducer<TR>(a, tile);
  const bool folds = reducer || (ALL && waits);
  // The group copy of the published inv this workgroup polls: per column one
  // 64-bit word (mark in the high half, the fp32 bits of inv in the low half).
  const unsigned long long* inv_copy = reinterpret_cast<const unsigned long long*>(
      a.ssq + epi_inv_off(a.epi_tiles) + (int64_t)(t16 % kEpiGroups) * kEpiRecordWords);
  // A tile that leaves its rows to the reducing workgroup has its out at the
  // coherence point in every compute wave before its record goes out.
  if (!waits) wait_vm_all();
  if (folds && wave == 0 && lane == 0) s_ctl[2] = 0u;
  __syncthreads();  // E1b
  if (wave == 0 && lane < a.B) {
    const unsigned long long tag = mark | (waits ? 0u : kEpiLeft);
#pragma unroll
    for (int h = 0; h < SUB; ++h) {
      if (t16 + h < a.epi_tiles) {
        float part = 0.0f;
        for (int r = 0; r < kBigTile; ++r) part = part + zz[(h * kBigTile + r) * 16 + lane];
        __hip_atomic_store(epi_record(a, t16 + h) + lane, (tag << 32) | __float_as_uint(part),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (!reducer && !waits) return;

  if (folds) {
    fold_records(a, mark, tile * (TR / kFlagRows), wave, lane, nt, wsum, s_inv, s_ctl,
                 TR > kBigTile);  // contains E3
    if (reducer && wave == 0) {
      // Every group's copy, one self-validating 64-bit word per column (so no
      // wait has to separate the values from a flag): P = B rounded up to a
      // power of two lanes per copy, consecutive lanes on consecutive words.
      const int lp = a.B <= 1 ? 0 : 32 - __builtin_clz((unsigned)(a.B - 1));  // log2 P
      const int c = lane & ((1 << lp) - 1);
      const unsigned long long word =
          ((unsigned long long)mark << 32) | __float_as_uint(s_inv[min(c, a.B - 1)]);
      if (!ALL && c < a.B) {
        for (int g = lane >> lp; g < kEpiGroups; g += 64 >> lp)
          __hip_atomic_store(reinterpret_cast<unsigned long long*>(
                                 a.ssq + epi_inv_off(a.epi_tiles) + (int64_t)g * kEpiRecordWords) +
                                 c,
                             word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (a.inv_rms && lane < a.B) a.inv_rms[lane] = s_inv[lane];
    }
  } else {
    if (wave == 0) {
      // Lane c < B polls column c's word until every column shows this call's
      // mark; its low half is then inv.  The reducing workgroup may itself
      // sit in its bounded peer wait and then in its bounded record wait:
      // allow four times the timeout.
      const uint64_t start = wall_clock64();
      float inv = __builtin_nanf("");
      for (;;) {
        const unsigned long long w = __hip_atomic_load(
            &inv_copy[min(lane, a.B - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool seen = lane >= a.B || (uint32_t)(w >> 32) == mark;
        if (__ballot(!seen) == 0) {
          inv = __uint_as_float((uint32_t)w);
          break;
        }
        if (wall_clock64() - start > 4 * a.timeout_ticks + 2000000ull) {
          if (lane == 0) {
            atomicOr(a.pad + kHdrErrorBits, kErrEpiWait);
            atomicMin(a.pad + kHdrEpiWaitTile, (uint32_t)(tile * (TR / kFlagRows)));
          }
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (lane < a.B) s_inv[lane] = inv;
    }
    __syncthreads();  // E3: inv in LDS (NaN if the wait expired)
  }
  __syncthreads();  // E4: inv in LDS
#pragma unroll
  for (int e = 0; e < OPL; ++e) {
    if (live[e]) {
      float v = z[e] * s_inv[b];
      if (a.rms_w) v = v * a.rms_w[row0 + n[e]];
      if (!ok[e]) v = __builtin_nanf("");
      store_y(a, (row0 + n[e]) * a.B + b, v);
    }
  }
  if (!reducer) return;

  // The reducing workgroup: the rows of every other tile tagged kEpiLeft in
  // this call (in the common case, where every tile saw all tiles started,
  // there are none).  Thread j takes tiles j, j + nt, ...; a tile's outputs
  // go four at a time, all loads of a batch before its stores.  The tags and
  // outputs are read only after the fold saw every record (E3, E4).
  constexpr int kBatch = 4;
  const int64_t NB = a.N * a.B;
  for (int t = wave * 64 + lane; t < a.epi_tiles; t += nt) {
    if (t / SUB == tile) continue;  // this workgroup's own rows
    const uint32_t tag = (uint32_t)(__hip_atomic_load(epi_record(a, t), __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) >> 32);
    if (tag != (mark | kEpiLeft)) continue;
    const int64_t lo = (int64_t)t * kBigTile * a.B;
    const int64_t hi = min(NB, lo + (int64_t)kBigTile * a.B);
    for (int64_t i0 = lo; i0 < hi; i0 += kBatch) {
      float ov[kBatch], bv[kBatch], wv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t i = min(i0 + u, hi - 1);
        const int64_t r = i / a.B;
        ov[u] = load_coherent(&a.out[i]);
        bv[u] = a.bias ? a.bias[r] : 0.0f;
        wv[u] = a.rms_w ? a.rms_w[r] : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t i = i0 + u;
        if (i < hi) {
          const int c = (int)(i % a.B);
          float v = (ov[u] + bv[u]) * s_inv[c];
          if (a.rms_w) v = v * wv[u];
          store_y(a, i, v);
        }
      }
    }
  }
}

// One A chunk (16 bytes) of each of the lane's R rows, at byte offset
// voff[s] + soff, through the buffer resource over A.  Rows past N, and the
// last row's chunks past the end of A, read zeros; other chunks past a row's
// end read the next row's data, which mac_chunk pairs with a zero x chunk (A
// is finite), so no load is masked.
template <int R>
__device__ __forceinline__ void load_chunk(uint4 (&av)[R], __amdgpu_buffer_rsrc_t ra,
                                           const uint32_t (&voff)[R], uint32_t soff) {
#pragma unroll
  for (int s = 0; s < R; ++s) av[s] = buf_load16(ra, voff[s] + soff);
}

// acc[s][b] += <A chunk of row s, x chunk c of batch b>.  x chunks live at
// lds_x[b * C + c]; lds_x[zidx] holds a zero chunk used for c >= C.
template <bool MASKED, int B, int R>
__device__ __forceinline__ void mac_chunk(float (&acc)[R][B], const uint4 (&av)[R],
                                          const uint4* lds_x, int C, int zidx, int c) {
  uint4 xv[B];
#pragma unroll
  for (int b = 0; b < B; ++b) xv[b] = lds_x[(MASKED && c >= C) ? zidx : b * C + c];
#pragma unroll
  for (int s = 0; s < R; ++s)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[s][b] = dot8(av[s], xv[b], acc[s][b]);
}

// Chunk slot of stream step j with the tile's rotation rot < NCH.
template <int NCH>
__device__ __forceinline__ int rotated(int j, int rot) {
  const int t = j + rot;
  return t >= NCH ? t - NCH : t;
}

// The lane's chunks as a stream with D chunks in flight: step j handles
// chunk li + rotated(j) * G of each row, ring[j % D] holds it, steps 0..D-1
// were issued before the LDS barrier.  A scheduling barrier closes each step
// (PIN): left free, the scheduler has hoisted later steps' x reads and sunk
// the refills behind them, draining the ring (twice the time on B = 8 rows
// of 224 chunks; after an unrelated change elsewhere in the kernel, the
// two-shot call on the 70B-class shape 14.7 against 12.4 us, the 8B
// down_proj at B = 4 5.71 against 5.41).  NCH > 0: exactly NCH chunks, fully
// unrolled, starting at the tile's rotation rot; NCH == 0: nch chunks in
// order, unrolled by D.
template <bool MASKED, int NCH, int D, int B, int G, int R, bool PIN>
__device__ __forceinline__ void valu_stream(float (&acc)[R][B], uint4 (&ring)[D][R],
                                            __amdgpu_buffer_rsrc_t ra, const uint32_t (&voff)[R],
                                            const uint4* lds_x, int C, int zidx, int li, int nch,
                                            int rot) {
  if constexpr (NCH > 0) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      mac_chunk<MASKED, B, R>(acc, ring[j % D], lds_x, C, zidx, li + rotated<NCH>(j, rot) * G);
      if (j + D < NCH)
        load_chunk<R>(ring[j % D], ra, voff, (uint32_t)(rotated<NCH>(j + D, rot) * G) * 16u);
      if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);  // the refill stays in its step
    }
  } else {
    for (int j0 = 0; j0 < nch; j0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int j = j0 + u;
        if (j < nch) {
          mac_chunk<MASKED, B, R>(acc, ring[u], lds_x, C, zidx, li + j * G);
          if (j + D < nch) load_chunk<R>(ring[u], ra, voff, (uint32_t)((j + D) * G) * 16u);
        }
        if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// VALU path, B <= 8.  NW compute waves plus one communication wave.  Each
// compute wave holds 64/G row groups of R rows; a row group of G lanes walks
// one row in 16-byte chunks li, li+G, ... as a stream with D chunks in flight
// per lane (the memory system accepts requests only as fast as it serves
// them, so a wave that issued everything up front would sit blocked at issue
// while its data arrives).  The compute waves first issue their share of x
// (XPT chunks per thread, into registers) and the first D chunks of A, then
// write x to LDS and pass the LDS barrier after only D chunks' worth of A
// loads (the compiler interleaves the two; forcing every x load ahead of the
// A loads measured slower, with all workgroups hitting the same x lines at
// once).  WPE is the occupancy (waves per SIMD) the register budget must
// allow.  NCH > 0 builds a fully unrolled instance for
// exactly NCH chunks per lane; MASKED instances zero chunks past the row end.
// TR = NW * (64 / G) * R rows per workgroup (4 or 16; the fused epilogue runs
// on 16).  XM: XCD-contiguous tile order (block_tile).
// LDS: x chunks [b][c], one zero chunk, one sink chunk, then the peer tile.
template <int B, int G, int R, int NW, int NCH, int D, int XPT, int WPE, bool MASKED, bool TS,
          bool XM, int DT, int EPI>
__global__ __launch_bounds__((NW + 1) * 64, WPE) void gemv_ar_valu(GemvArgs args) {
  const GemvArgs a = typed_args<DT>(args);
  constexpr int NT = NW * 64;
  constexpr int GPW = 64 / G;
  constexpr int TR = NW * GPW * R;
  static_assert(TR == kBigTile || TR == kFlagRows, "16-row or 4-row tiles");
  constexpr int V = R * B;
  static_assert(V <= G, "one owner lane per output of a row group");

  extern __shared__ uint4 lds_x[];
  __shared__ uint32_t s_ctl[kCtlWords];
  __shared__ unsigned long long s_epi_k;  // the epilogue's call index

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = block_tile<XM>();
  const int C = a.C;
  const int xchunks = B * C;
  const int zidx = xchunks;  // zero chunk; xchunks + 1 is the sink
  float* pe = reinterpret_cast<float*>(lds_x + xchunks + 2);
  float* elds = pe + a.W * TR * B + 1;  // the epilogue's LDS

  // The one-shot kernels with B <= 4 sum out before publishing (see
  // publish_and_reduce): the 8-wave tier from the communication wave's peer
  // tile, which it marks in s_ctl[8] (70B-class shape 12.06 against 12.20 us
  // with own loads), the others from peer values each lane loads itself
  // (from the tile: W=2 case 3.37 against 2.92 us, o_proj 4.04 against 3.46).
  // At B = 8 either measured slower than summing after B2 (8B down_proj shape
  // 6.16 against 5.85 us with own loads), so larger batches do that.
  constexpr bool kEarlyOut = !TS && B <= 4;
  // Every step of the A stream pinned (valu_stream), except in the 8-wave
  // tier at B = 8, where the pins make the registers spill.
  constexpr bool kPinSteps = !(G == 64 && NW == 8 && B == 8);
  constexpr bool kPeersFromTile = kEarlyOut && NW == 8;
  constexpr bool kOwnPeers = kEarlyOut && !kPeersFromTile;
  if (wave == NW) {
    comm_wave<TS, TR, !kOwnPeers, EPI>(a, lane, tile, pe, s_ctl, &s_epi_k);
    return;
  }

  const int grp = lane / G;
  const int li = lane % G;
  const int nloc0 = (wave * GPW + grp) * R;  // first local row of this row group
  const int64_t row0 = tile * TR + nloc0;
  const int nch = NCH > 0 ? NCH : (C + G - 1) / G;
  // The 4-row tiles start their rows at chunk step tile % NCH, so that the
  // first loads of neighbouring workgroups do not all fall at the same
  // offsets (Llama-3-8B o_proj shape: 3.45 against 3.51 us per call; on the
  // 16-row tiers it measured 3-5 % slower, so they start at 0).
  const int rot = (NCH > 0 && TR == kFlagRows) ? (int)(tile % NCH) : 0;

  const uint4* xg = reinterpret_cast<const uint4*>(a.x);
  __syncthreads();  // B0
  uint4 xr[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) xr[i] = xg[min(tid + i * NT, xchunks - 1)];

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(a.N * C * 16));
  uint32_t voff[R];
#pragma unroll
  for (int s = 0; s < R; ++s) voff[s] = ((uint32_t)(row0 + s) * (uint32_t)C + li) * 16u;
  uint4 ring[D][R];
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (NCH > 0 ? u < NCH : u < nch)
      load_chunk<R>(ring[u], ra, voff, (uint32_t)((NCH > 0 ? rotated<NCH>(u, rot) : u) * G) * 16u);

#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int idx = tid + i * NT;
    lds_x[idx < xchunks ? idx : xchunks + 1] = xr[i];  // out-of-range lanes: sink
  }
  for (int idx = tid + XPT * NT; idx < xchunks; idx += NT) lds_x[idx] = xg[idx];
  if (tid == 0) {
    lds_x[zidx] = make_uint4(0u, 0u, 0u, 0u);
    s_ctl[8] = 0u;
  }
  __syncthreads();  // B1
  const uint32_t state = s_ctl[1];
  // Every peer published at the start (one-shot call, B <= 4): each lane uses the
  // peer values of the output it will own (lane li < V: row nloc0 + li / B,
  // column li % B; other lanes repeat the last owner's addresses), loaded
  // here, after the flags were seen (B1): they queue behind this wave's A
  // loads and land as the stream ends.  The loads are unconditional (ranks
  // past W - 1 repeat rank W - 1's word, and when a peer had not published
  // the values are never used), so no branch join forces an early wait.
  const bool own_peers = kEarlyOut && state == kPeersReady;
  // Output o of the row group (row nloc0 + o / B, column o % B) ends in lanes
  // [o << SH, (o + 1) << SH) of the group (reduce-scatter); the first of them
  // owns it.
  constexpr int VP = pow2_at_least(V);
  constexpr int SH = log2_exact(G) - log2_exact(VP);
  const int vidx = min(li >> SH, V - 1);
  const bool vown = (li & ((1 << SH) - 1)) == 0 && (li >> SH) < V;
  const int64_t NB = a.N * a.B;
  const int64_t oi = min((row0 + vidx / B) * a.B + vidx % B, NB - 1);
  uint32_t pvb[kMaxW];
  if constexpr (kOwnPeers) {
#pragma unroll
    for (int r = 0; r < kMaxW; ++r) pvb[r] = load_slot_bits(a, min(r, a.W - 1) * NB + oi);
  } else {
#pragma unroll
    for (int r = 0; r < kMaxW; ++r) pvb[r] = 0u;
  }

  float acc[R][B];
#pragma unroll
  for (int s = 0; s < R; ++s)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[s][b] = 0.0f;
  valu_stream<MASKED, NCH, D, B, G, R, kPinSteps>(acc, ring, ra, voff, lds_x, C, zidx, li, nch,
                                                 rot);
  float pv[kMaxW];
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) pv[r] = slot_value(a, min(r, a.W - 1) * NB + oi, pvb[r]);

  // The V totals of the row group by one reduce-scatter (8B down_proj shape,
  // B = 8: 5.74 against 6.00 us per call with a full group sum per output).
  float vv[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) vv[i] = i < V ? acc[i / B][i % B] : 0.0f;
  float yv;
  if constexpr (G == 64)
    yv = reduce_scatter64<VP>(vv, lane);
  else
    yv = reduce_scatter32<VP>(vv, lane);
  if (kPeersFromTile && own_peers) {
    // The communication wave marks the peer tile stored without waiting for
    // the compute waves, so this wait ends.
    while (__hip_atomic_load(&s_ctl[8], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u)
      __builtin_amdgcn_s_sleep(1);  // acquire: the peer tile's LDS loads below stay after it
    const int idx = (nloc0 + vidx / B) * B + vidx % B;
#pragma unroll
    for (int r = 0; r < kMaxW; ++r) pv[r] = pe[min(r, a.W - 1) * (TR * B) + idx];
  }
  const int n[1] = {nloc0 + vidx / B};
  const bool own[1] = {vown};
  const float y[1] = {yv};
  publish_and_reduce<B, 1, TS, TR, EPI>(a, tile, n, vidx % B, own, y, pe, elds, s_ctl, &s_epi_k,
                                   state, wave, lane, NT, own_peers, pv);
}

// Long rows (C > 224 chunks, B <= 8), the plain one-shot call.  One
// workgroup of kLongWaves waves owns kLongRows = 32 rows; wave w takes rows
// 2w and 2w + 1 of the tile, a full wave per row: lane l streams chunks
// l, l + 64, ... of both rows with D chunk steps in flight.  Every x load of
// the workgroup goes out ahead of every A load (a scheduling barrier keeps
// that order; x is small and read by every workgroup, so it returns first,
// and the workgroup barrier that publishes x in LDS then waits for x alone,
// never for A).  Wave 0 also runs the signal-pad protocol: its flag loads go
// out before anything else, it takes the start decision (comm_decide) before
// that barrier, and after the publish it raises the tile's flags (and, if a
// peer had not published at the start, waits for it).  The 2 B partial sums
// of a lane are combined across the wave with one reduce-scatter, which
// leaves each output in one aligned lane group; its first lane loads that
// output's peer values right after the barrier (they queue behind the A
// stream), sums out in rank order, publishes y and stores out.
// Measured on the 70B-class down_proj shape (cold inputs, no protocol):
// 10.55 us per call against 10.9-12.0 us for 16-row workgroups of 8 waves
// with 2-7 steps in flight or x staged by LDS DMA (whose LDS writes the
// compiler orders behind every outstanding load), and against 9.9 us for a
// plain read of the same rows.
constexpr int kLongWaves = 16;
constexpr int kLongRows = 2 * kLongWaves;
constexpr int kLongCtlWords = 4 + kLongRows / kFlagRows;  // s_ctl[4 + q]: epoch of flag tile q


template <int B, int NCH, int D, int XPT, bool MASKED, int DT>
__global__ __launch_bounds__(kLongWaves * 64, kLongWaves / 4) void gemv_ar_long(GemvArgs args) {
  const GemvArgs a = typed_args<DT>(args);
  constexpr int R = 2;
  constexpr int NT = kLongWaves * 64;
  constexpr int TR = kLongRows;
  constexpr int V = R * B;                 // outputs of a wave: row s, column b at s * B + b
  constexpr int VP = pow2_at_least(V);     // padded for the reduce-scatter
  constexpr int SH = 6 - log2_exact(VP);   // output o sits in lanes [o << SH, (o + 1) << SH)
  static_assert(kLongRows / kFlagRows * kMaxW <= 64, "one wave-0 lane per (flag tile, rank)");

  extern __shared__ uint4 lds_x[];         // x chunks [b][c], one zero chunk, one sink chunk
  __shared__ uint32_t s_ctl[kLongCtlWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const FlagSpan fs = flag_span<TR>(a, tile);
  const int C = a.C;
  const int xchunks = B * C;
  const int zidx = xchunks;
  const int nch = NCH > 0 ? NCH : (C + 63) / 64;

  // Protocol state first: wave 0's flag loads lead every other load of the wave.
  uint32_t fl = 0;
  if (wave == 0) fl = load_flag(a, fs, lane);
  __builtin_amdgcn_sched_barrier(0);

  // x into registers (XPT <= 8 chunks per thread; indexes past x repeat the
  // last chunk and are written to the sink), then A.  Named registers, not
  // an array: across the scheduling barrier an array was kept in scratch.
  static_assert(XPT >= 1 && XPT <= 8, "x staged in at most 8 chunks per thread");
  const uint4* xg = reinterpret_cast<const uint4*>(a.x);
  uint4 x0, x1, x2, x3, x4, x5, x6, x7;
#define GSA_X_LOAD(k) \
  if constexpr (XPT > k) x##k = xg[min(tid + k * NT, xchunks - 1)];
  GSA_X_LOAD(0) GSA_X_LOAD(1) GSA_X_LOAD(2) GSA_X_LOAD(3)
  GSA_X_LOAD(4) GSA_X_LOAD(5) GSA_X_LOAD(6) GSA_X_LOAD(7)
#undef GSA_X_LOAD
  __builtin_amdgcn_sched_barrier(0);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(a.N * C * 16));
  const int64_t row0 = tile * TR + wave * R;
  uint32_t voff[R];
#pragma unroll
  for (int s = 0; s < R; ++s) voff[s] = ((uint32_t)(row0 + s) * (uint32_t)C + lane) * 16u;
  uint4 ring[D][R];
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (NCH > 0 ? u < NCH : u < nch) load_chunk<R>(ring[u], ra, voff, (uint32_t)u * 1024u);

  if (wave == 0) comm_decide<false, TR>(a, lane, tile, fs, fl, s_ctl);
#define GSA_X_PUT(k)                                    \
  if constexpr (XPT > k) {                              \
    const int idx = tid + k * NT;                       \
    lds_x[idx < xchunks ? idx : xchunks + 1] = x##k;    \
  }
  GSA_X_PUT(0) GSA_X_PUT(1) GSA_X_PUT(2) GSA_X_PUT(3)
  GSA_X_PUT(4) GSA_X_PUT(5) GSA_X_PUT(6) GSA_X_PUT(7)
#undef GSA_X_PUT
  if (tid == 0) lds_x[zidx] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();  // B1: x in LDS, the start decision in s_ctl
  const uint32_t state = s_ctl[1];

  // The output this lane group owns: o = lane >> SH (row o / B, column o % B).
  const int o = min(lane >> SH, V - 1);
  const bool owner = (lane & ((1 << SH) - 1)) == 0 && (lane >> SH) < V;
  const int64_t orow = row0 + o / B;
  const int64_t NB = a.N * a.B;
  const int64_t oi = min(orow * B + o % B, NB - 1);
  // Peer values of that output, loaded after the flags were seen (B1) when
  // every peer had published then; the loads are unconditional (ranks past
  // W - 1 repeat rank W - 1's word) and their values unused otherwise.  They
  // queue behind the lane's first A steps.  (Issued instead right behind the
  // lane's last A load, with each refill pinned to its step, they measured
  // no faster: 11.93 against 11.86 us per call on the 70B-class shape.)
  uint32_t pv[kMaxW];
#pragma unroll
  for (int r = 0; r < kMaxW; ++r) pv[r] = load_slot_bits(a, min(r, a.W - 1) * NB + oi);

  float acc[R][B];
#pragma unroll
  for (int s = 0; s < R; ++s)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[s][b] = 0.0f;
  valu_stream<MASKED, NCH, D, B, 64, R, false>(acc, ring, ra, voff, lds_x, C, zidx, lane, nch, 0);

  float v[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) v[i] = i < V ? acc[i / B][i % B] : 0.0f;
  const float y = reduce_scatter64<VP>(v, lane);

  const bool live = owner && orow < a.N;
  const float yp = publish_value(a, y);  // y as published: the own term of the sum
  float outv = 0.0f;
  if (state == kPeersReady) {
    // out = ((0 + s_0) + s_1) ... + s_{W-1}, the own term being y as
    // published; ranks past W - 1 add +0 (acc is never -0).
#pragma unroll
    for (int r = 0; r < kMaxW; ++r)
      outv = outv + (r < a.W ? (r == a.rank ? yp : slot_value(a, r * NB + oi, pv[r])) : 0.0f);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (state != kBadOwnRow && live) store_slot(a, a.rank * NB + oi, yp);
  __builtin_amdgcn_sched_barrier(0);
  if (state == kPeersReady) {
    if (live) store_out(a, oi, outv);
    wait_vm_le<1>();  // the published value is at the coherence point (stores complete in order)
  } else {
    wait_vm_all();
  }
  __syncthreads();  // B2: every published value of the tile is at the coherence point
  if (state != kBadOwnRow && wave == 0 && lane < fs.nf)
    store_flag(flag_ptr(a, a.rank, fs.f0 + lane), s_ctl[4 + lane]);
  if (state == kMustWait) {
    // A peer had not published at the start: wait for it (bounded), then
    // load the peer values of the complete flag tiles and write out.
    if (wave == 0) {
      const uint32_t done = wait_peers<false, TR>(a, lane, tile, fs, s_ctl);
      if (lane == 0) s_ctl[0] = done;
    }
    __syncthreads();  // B3
    const uint32_t done = s_ctl[0];
    const int q = (int)(orow - tile * TR) / kFlagRows;
    if (live && ((done >> q) & 1u)) {
      float acc2 = 0.0f;
#pragma unroll
      for (int r = 0; r < kMaxW; ++r) {
        if (r < a.W) acc2 = acc2 + (r == a.rank ? yp : load_slot(a, r * NB + oi));
      }
      store_out(a, oi, acc2);
    }
  }
}

// MFMA epilogue: each wave's 16 x 16 partial goes to red[wave][n][b]; after
// B1 wave w sums rows 4w .. 4w+3 over the waves in wave order (lane l: row
// 4w + (l >> 4), column l & 15), publishes them and reduces.
template <int NW, bool TS, int EPI>
__device__ __forceinline__ void mfma_finish(const GemvArgs& a, int64_t tile, int wave, int lane,
                                            f32x4_t acc, float* red, const float* pe,
                                            float* elds, uint32_t* s_ctl,
                                            const unsigned long long* s_epi_k) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    red[(wave * kBigTile + 4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[e];
  __syncthreads();  // B1: every partial in LDS, the decision in s_ctl
  const uint32_t state = s_ctl[1];
  const int nl = 4 * wave + (lane >> 4);
  const int bl = lane & 15;
  float y = red[nl * 16 + bl];
#pragma unroll
  for (int w = 1; w < NW; ++w) y = y + red[(w * kBigTile + nl) * 16 + bl];
  const int n[1] = {nl};
  const bool own[1] = {bl < a.B};
  const float yv[1] = {y};
  const float no_pv[kMaxW] = {};
  publish_and_reduce<GSA_MAX_B, 1, TS, kBigTile, EPI>(a, tile, n, bl, own, yv, pe, elds, s_ctl,
                                                 s_epi_k, state, wave, lane, NW * 64, false,
                                                 no_pv);
}

// MFMA path, 8 < B <= 16 (batch padded to 16 with zeros).  The tile's 16 rows
// form the A operand of v_mfma_f32_16x16x32_bf16, x (16 batches x 32 k) the
// B operand from LDS.  The NW compute waves split the k-steps (32 k each).
// Each wave copies the x columns of its own k-steps from memory straight
// into LDS (no registers, no barrier: it waits for its own copies), then
// streams its A chunks with D steps in flight per lane.  Operand layout per
// lane l: A row (l & 15), B column (l & 15), k-chunk (l >> 4) of the step's
// four 8-element chunks; result rows 4*(l >> 4) + e, column (l & 15).  x
// chunks past a row's end come from the zero column C, batch rows >= B are
// zero; A chunks there read other data or zeros, which meet those zeros (A
// is finite).  The per-wave 16 x 16 fp32 partials are summed in wave order
// through LDS.  One more wave runs the signal-pad protocol.
// LDS: x [16][C + 1] chunks (column C zero); NW 16 x 16 partials; peer tile.
template <int NW, int D, bool TS, int DT, int EPI>
__global__ __launch_bounds__((NW + 1) * 64, 3) void gemv_ar_mfma(GemvArgs args) {
  const GemvArgs a = typed_args<DT>(args);
  static_assert(NW * 4 == kBigTile, "each compute wave finishes 4 rows of the tile");
  extern __shared__ uint4 lds[];
  __shared__ uint32_t s_ctl[kCtlWords];
  __shared__ unsigned long long s_epi_k;  // the epilogue's call index

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const int C = a.C;
  const int CP = C + 1;  // padded LDS row: the 16 batch rows of one chunk hit distinct banks
  float* red = reinterpret_cast<float*>(lds + 16 * CP);
  float* pe = red + NW * kBigTile * 16;
  float* elds = pe + a.W * kBigTile * a.B + 1;  // the epilogue's LDS

  if (wave == NW) {
    comm_wave<TS, kBigTile, true, EPI>(a, lane, tile, pe, s_ctl, &s_epi_k);
    return;
  }

  const int64_t row0 = tile * kBigTile;
  const int steps = (C + 3) / 4;
  const int per_wave = (steps + NW - 1) / NW;
  const int s_begin = wave * per_wave;
  const int n_steps = max(0, min(steps, s_begin + per_wave) - s_begin);
  // This wave's chunks of every row: [c_begin, c_end), all < C.
  const int c_begin = min(4 * s_begin, C);
  const int c_end = min(4 * (s_begin + n_steps), C);

  __syncthreads();  // B0
  // x columns [c_begin, c_end) of batch rows < B, 64 chunks per copy.
  const uint4* xg = reinterpret_cast<const uint4*>(a.x);
  for (int c0 = c_begin; c0 < c_end; c0 += 64) {
    if (c0 + lane < c_end) {
      for (int b = 0; b < a.B; ++b) lds_dma16(xg + (int64_t)b * C + c0 + lane, lds + b * CP + c0);
    }
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(a.N * C * 16));
  const int kq = lane >> 4;
  const uint32_t a_row = ((uint32_t)(row0 + (lane & 15)) * (uint32_t)C + kq) * 16u;
  const uint32_t kOutOfRange = 0x80000000u;  // past any A buffer: reads zeros
  // A chunk of the wave's step j; steps past n_steps read zeros.  Every load
  // is issued unconditionally, so the outstanding-load counts are static.
  auto a_off = [&](int j) {
    return j < n_steps ? a_row + (uint32_t)(s_begin + j) * 64u : kOutOfRange;
  };
  uint4 ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) ring[u] = buf_load16(ra, a_off(u));
  // This wave's x copies were issued before its D ring loads: once at most D
  // loads are outstanding they have landed, before any other LDS access.
  wait_vm_le<D>();
  // Zeros this wave's steps may read: batch rows >= B and the column C.
  for (int c = c_begin + lane; c < c_end; c += 64)
    for (int b = a.B; b < 16; ++b) lds[b * CP + c] = make_uint4(0u, 0u, 0u, 0u);
  if (lane < 16) lds[lane * CP + C] = make_uint4(0u, 0u, 0u, 0u);

  // Whole blocks of D steps; a step past n_steps multiplies zeros from A by
  // the zero column of x and adds +0 to an accumulator that is never -0.
  // A block first reads its D x chunks from LDS, then each step runs its
  // MFMA and refills its ring slot, in that order (the scheduling barrier
  // keeps each refill next to its MFMA instead of letting a block's refills
  // sink to its end).
  const int xrow = (lane & 15) * CP;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < n_steps; j0 += D) {
    uint4 xv[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int j = j0 + u;
      const int chunk = 4 * (s_begin + j) + kq;
      xv[u] = lds[xrow + (j < n_steps && chunk < C ? chunk : C)];
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ring[u]),
                                                    __builtin_bit_cast(bf16x8_t, xv[u]), acc, 0,
                                                    0, 0);
      ring[u] = buf_load16(ra, a_off(j0 + u + D));
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  mfma_finish<NW, TS, EPI>(a, tile, wave, lane, acc, red, pe, elds, s_ctl, &s_epi_k);
}

// MFMA path for x beyond the LDS bound (8 < B <= 16, 16 * (C + 1) chunks over
// GSA_MAX_X_LDS_BYTES): as gemv_ar_mfma, but the B operand is read from
// memory (x stays in L2; rows >= B and chunks past a row's end read zeros
// through out-of-range offsets), streamed with A, D steps in flight.  The
// wave's steps start at a rotation that differs between the workgroups of
// one XCD so that they do not all read the same lines of x at once.
// LDS: NW 16 x 16 partials, then the peer tile.
template <int NW, int D, bool TS, int DT, int EPI>
__global__ __launch_bounds__((NW + 1) * 64, 3) void gemv_ar_mfma_xmem(GemvArgs args) {
  const GemvArgs a = typed_args<DT>(args);
  static_assert(NW * 4 == kBigTile, "each compute wave finishes 4 rows of the tile");
  extern __shared__ uint4 lds[];
  __shared__ uint32_t s_ctl[kCtlWords];
  __shared__ unsigned long long s_epi_k;  // the epilogue's call index

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const int C = a.C;
  float* red = reinterpret_cast<float*>(lds);
  float* pe = red + NW * kBigTile * 16;
  float* elds = pe + a.W * kBigTile * a.B + 1;  // the epilogue's LDS

  if (wave == NW) {
    comm_wave<TS, kBigTile, true, EPI>(a, lane, tile, pe, s_ctl, &s_epi_k);
    return;
  }

  const int64_t row0 = tile * kBigTile;
  const int steps = (C + 3) / 4;
  const int per_wave = (steps + NW - 1) / NW;
  const int s_begin = wave * per_wave;
  const int n_steps = max(0, min(steps, s_begin + per_wave) - s_begin);
  const int rot = n_steps > 0 ? (int)((tile >> 3) % n_steps) : 0;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, (uint32_t)(a.N * C * 16));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(a.B * C * 16));
  const int kq = lane >> 4;
  const int l16 = lane & 15;
  const uint32_t a_row = ((uint32_t)(row0 + l16) * (uint32_t)C + kq) * 16u;
  const uint32_t x_row = ((uint32_t)l16 * (uint32_t)C + kq) * 16u;  // past x for l16 >= B
  const uint32_t kOutOfRange = 0x80000000u;
  // The wave's j-th step in its rotated order; steps past n_steps read zeros.
  auto step_of = [&](int j) {
    const int p = j + rot;
    return s_begin + (p >= n_steps ? p - n_steps : p);
  };
  auto a_off = [&](int j) {
    return j < n_steps ? a_row + (uint32_t)step_of(j) * 64u : kOutOfRange;
  };
  auto x_off = [&](int j) {
    if (j >= n_steps) return kOutOfRange;
    const int st = step_of(j);
    return 4 * st + kq < C ? x_row + (uint32_t)st * 64u : kOutOfRange;
  };

  __syncthreads();  // B0
  uint4 ra_ring[D], rx_ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    ra_ring[u] = buf_load16(ra, a_off(u));
    rx_ring[u] = buf_load16_cached(rx, x_off(u));
  }

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = 0; j0 < n_steps; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ra_ring[u]),
                                                    __builtin_bit_cast(bf16x8_t, rx_ring[u]),
                                                    acc, 0, 0, 0);
      ra_ring[u] = buf_load16(ra, a_off(j0 + u + D));
      rx_ring[u] = buf_load16_cached(rx, x_off(j0 + u + D));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  mfma_finish<NW, TS, EPI>(a, tile, wave, lane, acc, red, pe, elds, s_ctl, &s_epi_k);
}

// One-GPU stand-in for a peer's zero-copy push (the fused-operators page:
// results written straight into peer memory, then signalled): one
// workgroup spins `delay_ticks` of device wall-clock time, stores `values`
// into slot `peer` with device-coherent stores, waits until every store of
// the workgroup is complete (vmcnt(0), then the barrier), and only then
// stores `epoch` into each of peer's flags.  The spin is bounded by its
// argument, so the kernel always ends.
__global__ __launch_bounds__(256) void peer_publish_kernel(float* slots, uint32_t* pad,
                                                           const void* values, int peer,
                                                           int64_t NB, int slot_bf16,
                                                           int row_stride, int64_t nflags,
                                                           uint32_t epoch, uint64_t delay_ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < delay_ticks) __builtin_amdgcn_s_sleep(32);
  const int64_t base = (int64_t)peer * NB;
  for (int64_t i = threadIdx.x; i < NB; i += blockDim.x) {
    if (slot_bf16)
      __hip_atomic_store(reinterpret_cast<uint16_t*>(slots) + base + i,
                         static_cast<const uint16_t*>(values)[i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      store_coherent(slots + base + i, static_cast<const float*>(values)[i]);
  }
  wait_vm_all();
  __syncthreads();  // every value is at the coherence point before any flag
  uint32_t* row = pad + GSA_PAD_HEADER_WORDS + (int64_t)peer * row_stride;
  for (int64_t t = threadIdx.x; t < nflags; t += blockDim.x) store_flag(row + flag_word(t), epoch);
}

// MFMA path with A staged through LDS: 8 < B <= 16, rows of exactly 256
// chunks, the one-shot call, plain or with the fused epilogue (the skinny
// GEMM; the epilogue takes the 16-row MFMA kernel's 16.0 to 15.2 us per
// call there: wave 0 counts the workgroup's two 16-row tiles started,
// reads the started counts right after its MFMAs, the partials' LDS holds
// the squares, and the producer waves join the epilogue's barriers).  One
// workgroup owns 32
// rows (two 16-row blocks of v_mfma_f32_16x16x32_bf16) with 4 consumer waves
// and 2 producer waves.  Consumer wave w owns chunks [64 w, 64 w + 64) of
// every row, in 8 stages of 8 chunks.  The producers copy A into LDS with
// direct-to-LDS loads, 4 stages in flight: each copy instruction reads 8 rows
// x 128 bytes (whole lines; the MFMA operand itself reads 64 bytes of each of
// 16 rows per instruction, half a line, which measured 8.3 us against 6.4
// for the same bytes read whole), laid out in 1 KB blocks with the chunk
// index XOR-ed with the row, so that a consumer's 16-row operand read hits
// 16 distinct banks.  Stage j is complete when its producer's counted wait
// returns; a plain s_barrier then hands it over (a barrier with a fence
// would wait for every copy in flight).  The consumers issue no A loads, so
// their LDS reads carry no wait for the copies; they load their x operands
// a stage at a time, two stages ahead (all of x at the start, 64 KB per
// workgroup at once, cost 1.1 us), and the peer values of their two outputs
// right behind their last x loads.  Wave 0 runs the signal-pad protocol and
// takes the start decision before the first stage barrier.  The waves'
// partials are summed in wave order through LDS; each consumer thread then
// owns two outputs, sums them with their peer values in rank order and
// publishes them (the long-row kernel's scheme).  Measured on the skinny
// GEMM (cold, per call): without the protocol 7.9 us against 9.6 for the
// same MFMAs with every lane loading its own A operands and all of x in
// registers; with it 9.0 against 10.4.  Each workgroup starts its walk over
// the 8 stages at a stage of its own ((t ^ (t >> 3)) mod 8 for tile t): 8.7
// against 9.05 us with every workgroup in the same order.  Not taken
// (same box, us per call): 5-7 stages in flight 9.3-9.6; a stage of 512
// contiguous bytes of each row 10.2-10.4; a stage of 16 whole 1 KB row
// pieces 10.1 (9.2 with the rotation); a workgroup's 4-row groups spread
// over the matrix instead of contiguous, no gain.
constexpr int kMfmaLCons = 4;     // consumer waves (MFMA)
constexpr int kMfmaLProd = 2;     // producer waves (A into LDS)
constexpr int kMfmaLRows = 32;
constexpr int kMfmaLStages = 8;   // stages per workgroup: 8 chunks of each consumer's 64
constexpr int kMfmaLInFlight = 4; // stages in LDS at once
constexpr int kMfmaLBlocks = kMfmaLCons * (kMfmaLRows / 8);  // 1 KB blocks per stage
constexpr int kMfmaLStageBytes = kMfmaLBlocks * 1024;
constexpr size_t kMfmaLLdsBytes = (size_t)kMfmaLInFlight * kMfmaLStageBytes +
                                  (size_t)kMfmaLCons * kMfmaLRows * 16 * sizeof(float);

// s_waitcnt vmcnt(n) for a count known only after unrolling (0 <= n <= 63).
template <int K>
__device__ __forceinline__ void wait_vm_le_n(int n) {
  if constexpr (K >= 0) {
    if (n == K)
      wait_vm_le<K>();
    else
      wait_vm_le_n<K - 1>(n);
  }
}

// The stage a workgroup of tile t starts its walk at: position j holds stage
// (j + rot) mod NS of the row, so that neighbouring workgroups, on one XCD
// (t >> 3) and across XCDs (t & 7), do not request the same offsets of their
// rows at once.  (Computed where it is used: kept in a register from the
// kernel's start, the same value measured 0.4 us slower per call, from a
// different schedule of the x loads.)
template <int NS>
__device__ __forceinline__ int lds_stage_rot(int64_t t) {
  return (int)((t ^ (t >> 3)) & (NS - 1));
}

template <int DT, int EPI>
__global__ __launch_bounds__((kMfmaLCons + kMfmaLProd) * 64) void gemv_ar_mfma_lds(GemvArgs args) {
  const GemvArgs a = typed_args<DT>(args);
  constexpr int RB = kMfmaLRows / 16;
  constexpr int NT = kMfmaLCons * 64;  // consumer threads
  constexpr int TR = kMfmaLRows;
  constexpr int OPT = TR * 16 / NT;    // outputs per consumer thread
  constexpr int NS = kMfmaLStages;
  constexpr int S = kMfmaLInFlight;
  constexpr int PER = kMfmaLBlocks / kMfmaLProd;  // copies per producer per stage
  constexpr int XPF = 2;                          // stages of x loaded ahead
  static_assert(PER * S <= 63, "a producer's copies in flight fit the vmcnt counter");
  static_assert(kMfmaLRows / kFlagRows * kMaxW <= 64, "one wave-0 lane per (flag tile, rank)");
  static_assert(NS > XPF, "the peer loads follow the last x loads");
  extern __shared__ __align__(16) unsigned char lds_a[];
  float* red = reinterpret_cast<float*>(lds_a + S * kMfmaLStageBytes);  // [wave][RB][16][16]
  __shared__ uint32_t s_ctl[kLongCtlWords];
  __shared__ unsigned long long s_epi_k;  // the fused epilogue's call index
  constexpr int SUB = TR / kBigTile;      // the epilogue's 16-row tiles per workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const FlagSpan fs = flag_span<TR>(a, tile);
  const int C = a.C;  // == 256
  const int64_t row0 = tile * TR;

  if (wave >= kMfmaLCons) {
    // Producer p: blocks b = 2 i + p of every stage; block b holds rows
    // 8 (b % 4) .. + 7 of consumer wave b / 4's 8 chunks; lane l copies row
    // l / 8, chunk (l % 8) ^ (l / 8) of it (rows past N repeat row N - 1).
    const int p = wave - kMfmaLCons;
    auto issue = [&](int j, int buf) {
      const int st = (j + lds_stage_rot<NS>(tile)) & (NS - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = 2 * i + p;
        const int64_t r = min(row0 + (b & 3) * 8 + (lane >> 3), a.N - 1);
        const int chunk = 64 * (b >> 2) + 8 * st + ((lane & 7) ^ (lane >> 3));
        lds_dma16<2>(a.A + (r * C + chunk) * 8, lds_a + buf * kMfmaLStageBytes + b * 1024);
      }
    };
#pragma unroll
    for (int j = 0; j < S; ++j) issue(j, j);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // stage j complete: only the copies of later stages may be in flight
      const int last = min(NS - 1, S - 1 + max(0, j - 1));
      wait_vm_le_n<63>((last - j) * PER);
      asm volatile("s_barrier" ::: "memory");  // stage j handed over
      if (j >= 1 && j - 1 + S < NS) issue(j - 1 + S, (j - 1) % S);  // the buffer of stage j - 1
    }
    __syncthreads();  // R: partials
    const uint32_t state = s_ctl[1];
    __syncthreads();  // B2
    if (state == kMustWait) __syncthreads();  // B3
    if constexpr (EPI) {
      __syncthreads();  // E1
      __syncthreads();  // E1b
      if (s_ctl[3] || epi_reducer<TR>(a, tile)) {  // a waiting tile, or the reducing workgroup
        __syncthreads();  // E3
        __syncthreads();  // E4
      }
    }
    return;
  }

  const int kq = lane >> 4;
  const int l16 = lane & 15;
  const uint32_t kOutOfRange = 0x80000000u;  // past any buffer: reads zeros

  uint32_t fl = 0;
  unsigned long long epi_before = 0;
  if (wave == 0) {
    fl = load_flag(a, fs, lane);
    // The fused epilogue: count the workgroup's 16-row tiles started (the
    // value is used once the protocol work is done).
    if constexpr (EPI) epi_before = epi_count_started(a, tile * SUB, SUB, lane);
  }
  __builtin_amdgcn_sched_barrier(0);

  // x: batch l16 (zeros past B), chunk 64 wave + 4 s + kq of MFMA step s.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(a.B * C * 16));
  auto x_off = [&](int j2) {  // MFMA step j2 = 2 j + m of position j: step s of the row
    const int s = 2 * (((j2 >> 1) + lds_stage_rot<NS>(tile)) & (NS - 1)) + (j2 & 1);
    return l16 < a.B ? ((uint32_t)l16 * (uint32_t)C + 64u * wave + 4u * s + kq) * 16u
                     : kOutOfRange;
  };
  uint4 xv[2 * NS];
#pragma unroll
  for (int s2 = 0; s2 < 2 * XPF; ++s2) xv[s2] = buf_load16_cached(rx, x_off(s2));

  if (wave == 0) comm_decide<false, TR>(a, lane, tile, fs, fl, s_ctl);

  const int64_t NB = a.N * a.B;
  int64_t oi[OPT];
  bool live[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + NT * i;
    const int64_t row = row0 + o / 16;
    const int b = o % 16;
    live[i] = b < a.B && row < a.N;
    oi[i] = min(row * a.B + min(b, a.B - 1), NB - 1);
  }
  uint32_t pv[OPT][kMaxW];

  f32x4_t acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    // this wave's reads of stage j - 1 are complete; stage j is in LDS
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + XPF < NS) {
#pragma unroll
      for (int m = 0; m < 2; ++m) xv[2 * (j + XPF) + m] = buf_load16_cached(rx, x_off(2 * (j + XPF) + m));
    }
    if (j == NS - 1 - XPF) {
      // The peer values, right behind the last x loads: unconditional
      // (clamped) loads, unused unless every peer had published at the start.
#pragma unroll
      for (int i = 0; i < OPT; ++i)
#pragma unroll
        for (int r = 0; r < kMaxW; ++r) pv[i][r] = load_slot_bits(a, min(r, a.W - 1) * NB + oi[i]);
    }
    const unsigned char* st = lds_a + (j % S) * kMfmaLStageBytes;
    uint4 av[2][RB];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 16 + l16;
        const int c = 4 * m + kq;  // chunk within the wave's 8 of this stage
        const int off = (wave * 4 + (row >> 3)) * 1024 + (row & 7) * 128 + ((c ^ (row & 7)) * 16);
        av[m][rb] = *reinterpret_cast<const uint4*>(st + off);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[m][rb]),
                                                          __builtin_bit_cast(bf16x8_t, xv[2 * j + m]),
                                                          acc[rb], 0, 0, 0);
  }
  // The fused epilogue's reading of the started counts, taken here so that
  // its round trip overlaps the publish (any tile counted by now has started).
  unsigned long long epi_now = 0;
  if constexpr (EPI) {
    if (wave == 0) epi_now = epi_started_load(a, lane);
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * RB + r) * 16 + 4 * kq + e) * 16 + l16] = acc[r][e];
  __syncthreads();  // R: every wave's partials in LDS, the start decision in s_ctl
  const uint32_t state = s_ctl[1];

  float yp[OPT], outv[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + NT * i;
    const int lr = o / 16, b = o % 16;
    float y = red[((0 * RB + lr / 16) * 16 + lr % 16) * 16 + b];
#pragma unroll
    for (int w = 1; w < kMfmaLCons; ++w) y = y + red[((w * RB + lr / 16) * 16 + lr % 16) * 16 + b];
    yp[i] = publish_value(a, y);  // y as published: the own term of the sum
    outv[i] = 0.0f;
    if (state == kPeersReady) {
#pragma unroll
      for (int r = 0; r < kMaxW; ++r)
        outv[i] = outv[i] +
                  (r < a.W ? (r == a.rank ? yp[i] : slot_value(a, r * NB + oi[i], pv[i][r])) : 0.0f);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (state != kBadOwnRow) {
#pragma unroll
    for (int i = 0; i < OPT; ++i)
      if (live[i]) store_slot(a, a.rank * NB + oi[i], yp[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // With the fused epilogue, out is stored device-coherently: the reducing
  // workgroup may read it back.
  auto put_out = [&](int64_t i, float v) {
    if constexpr (EPI)
      store_coherent(&a.out[i], v);
    else
      store_out(a, i, v);
  };
  bool okv[OPT];  // out of the output computed (its flag tile complete)
#pragma unroll
  for (int i = 0; i < OPT; ++i) okv[i] = state == kPeersReady;
  if (state == kPeersReady) {
#pragma unroll
    for (int i = 0; i < OPT; ++i)
      if (live[i]) put_out(oi[i], outv[i]);
    wait_vm_le<OPT>();  // the published values are at the coherence point (in-order completion)
  } else {
    wait_vm_all();
  }
  __syncthreads();  // B2: every published value of the tile is at the coherence point
  if (state != kBadOwnRow && wave == 0 && lane < fs.nf)
    store_flag(flag_ptr(a, a.rank, fs.f0 + lane), s_ctl[4 + lane]);
  if (state == kMustWait) {
    if (wave == 0) {
      const uint32_t done = wait_peers<false, TR>(a, lane, tile, fs, s_ctl);
      if (lane == 0) s_ctl[0] = done;
    }
    __syncthreads();  // B3
    const uint32_t done = s_ctl[0];
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int q = ((tid + NT * i) / 16) / kFlagRows;
      okv[i] = ((done >> q) & 1u) != 0;
      if (live[i] && okv[i]) {
        float acc2 = 0.0f;
#pragma unroll
        for (int r = 0; r < kMaxW; ++r)
          if (r < a.W) acc2 = acc2 + (r == a.rank ? yp[i] : load_slot(a, r * NB + oi[i]));
        outv[i] = acc2;
        put_out(oi[i], acc2);
      }
    }
  }
  if constexpr (EPI) {
    // Thread tid holds outputs tid + NT i: local row (tid + NT i) / 16,
    // column tid % 16.  The partials in `red` were all read before B2, so
    // the epilogue's LDS takes their place.
    if (wave == 0) epi_note_started(a, tile * SUB, epi_before, epi_now, lane, s_ctl, &s_epi_k);
    int n[OPT];
    bool own[OPT];
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      n[i] = (tid + NT * i) / 16;
      own[i] = (tid & 15) < a.B;
    }
    fused_epilogue<GSA_MAX_B, OPT, TR, false>(a, tile, n, tid & 15, own, live, outv, okv, red, s_ctl,
                                       &s_epi_k, wave, lane, NT);
  }
}

__global__ void pad_reset_kernel(uint32_t* pad, int W, int row_stride, uint32_t mask,
                                 uint32_t* epi, int64_t epi_words) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < epi_words) epi[i] = 0u;  // the epilogue's records, 1/rms copies and counts
  // Header, then 2W flag rows: rank r's slot flags (row r) and reduced-chunk
  // flags of the two-shot variant (row W + r).
  const int64_t total = GSA_PAD_HEADER_WORDS + 2 * (int64_t)W * row_stride;
  if (i >= total) return;
  uint32_t v;
  if (i < GSA_PAD_HEADER_WORDS) {
    v = (i == kHdrTimeoutKey || i == kHdrStateTile || i == kHdrEpiWaitTile) ? 0xFFFFFFFFu : 0u;
  } else {
    const int r = (int)((i - GSA_PAD_HEADER_WORDS) / row_stride) % W;
    v = ((mask >> r) & 1u) ? GSA_FLAG_PUBLISHED : 0u;
  }
  pad[i] = v;
}

constexpr int kMfmaWaves = 4;

// Whether the MFMA path stages x ([16][C + 1] chunks) in LDS.
bool mfma_x_in_lds(int C) { return (size_t)16 * (C + 1) * 16 <= GSA_MAX_X_LDS_BYTES; }

struct ValuChoice {
  const void* kernel;
  int threads;    // per workgroup (compute waves, plus the communication wave if the kernel has one)
  int tile_rows;  // rows per workgroup
  bool fixed_lds = false;  // dynamic LDS of a fixed size (lds_bytes), not from the shape
  size_t lds_bytes = 0;
};

constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// One tier: G lanes per row, R rows per row group, NW compute waves, D chunks
// in flight per lane, occupancy WPE.  C == G * NCH gets the fully unrolled
// exact instance; any other C the masked streaming instance.  XPT covers
// B * G * NCH chunks of x (at most 8 per thread; the rest of a longer x is
// staged by a plain loop).
template <int B, int G, int R, int NW, int NCH, int D, int WPE, bool TS, bool XM, int DT, int EPI>
ValuChoice valu_tier(int C) {
  constexpr int XPT0 = ceil_div(B * G * NCH, NW * 64);
  constexpr int XPT = XPT0 > 8 ? 8 : XPT0;
  constexpr int DE = D < NCH ? D : NCH;
  const void* k;
  if (C == G * NCH)
    k = reinterpret_cast<const void*>(
        &gemv_ar_valu<B, G, R, NW, NCH, DE, XPT, WPE, false, TS, XM, DT, EPI>);
  else
    k = reinterpret_cast<const void*>(
        &gemv_ar_valu<B, G, R, NW, 0, D, XPT, WPE, true, TS, XM, DT, EPI>);
  return {k, (NW + 1) * 64, NW * (64 / G) * R};
}

// The long-row kernel: an unrolled instance for rows of exactly 448 chunks
// (the 70B-class down_proj shard), a masked streaming one for the others;
// 4 chunk steps in flight (measured: 10.55 us on the 70B-class shape against
// 11.1 at 3 and 10.6-12.0 at 5-7, cold, without the protocol).
template <int B, int DT>
ValuChoice long_tier(int C) {
  constexpr int kExactNch = 7;
  constexpr int XPT = ceil_div(B * 64 * kExactNch, kLongWaves * 64);
  constexpr int D = 4;
  const void* k = C == 64 * kExactNch
                      ? reinterpret_cast<const void*>(&gemv_ar_long<B, kExactNch, D, XPT, false, DT>)
                      : reinterpret_cast<const void*>(&gemv_ar_long<B, 0, D, 8, true, DT>);
  return {k, kLongWaves * 64, kLongRows};
}

// VALU tiers by chunks per row C = Ks / 8 (plus the communication wave):
//   C <= 64, no epilogue: 4 rows per workgroup, 1 wave, half a wave per row,
//            2 x 2 rows (more, smaller workgroups: on the Llama-3-8B o_proj
//            shape 4.05 against 4.49 us per call with 16-row tiles)
//   C <= 64 : 16 rows, 4 waves, a full wave per row, 4 rows per wave
//   C <= 224: 16 rows, 4 waves, half a wave per row, 2 x 2 rows per wave
//   larger, plain call: the long-row kernel (32 rows, 16 waves)
//   larger, epilogue or two-shot: 16 rows, 8 waves, a full wave per row,
//            2 rows per wave
// (4-row tiles on the longer rows measured slower: 5.4-5.5 against 5.25 us on
// the 8B down_proj shape, 14.9 against 12.3 us on the 70B-class one.)  Tiles
// of rows up to C = 224 go to the XCDs in contiguous runs (block_tile).
// DT other than fp32 (bf16 slots or out) comes only with small tiles and
// one-shot: the instances it takes are the ones those calls reach.
template <int B, bool TS, int DT, int EPI>
ValuChoice valu_kernel(int C) {
  static_assert(!(DT != kDtF32 && (TS || EPI)), "element types are for the plain one-shot call");
  static_assert(!(TS && EPI), "no fused epilogue in the two-shot call");
  if constexpr (!EPI) {
    if (!TS && C > 224) return long_tier<B, DT>(C);
    if (C <= 64) return valu_tier<B, 32, 2, 1, 2, 2, 1, TS, true, DT, kEpiNone>(C);
  } else {
    // The fused epilogue counts 16-row tiles.
    if (C <= 64) return valu_tier<B, 64, 4, 4, 1, 1, 1, false, true, kDtF32, EPI>(C);
  }
  if constexpr (EPI == kEpiFoldAll) {
    return ValuChoice{nullptr, 0, 0};  // not reached: chosen for rows of at most 64 chunks
  } else {
    if (C <= 224) return valu_tier<B, 32, 2, 4, 7, 4, 1, TS, true, DT, EPI>(C);
    if constexpr (DT != kDtF32)
      return ValuChoice{nullptr, 0, 0};  // not reached: the plain call takes the long tier
    else
      return valu_tier<B, 64, 2, 8, 7, 3, 5, TS, false, kDtF32, EPI>(C);
  }
}

// EPI: the kernels of the fused epilogue, instances of their own, so that the
// plain and two-shot instances carry none of its code (the compiler's
// schedule of their A stream has moved with changes to it).
template <bool TS, int DT, int EPI>
ValuChoice pick_kernel(int B, int C) {
  switch (B) {
    case 1: return valu_kernel<1, TS, DT, EPI>(C);
    case 2: return valu_kernel<2, TS, DT, EPI>(C);
    case 3: return valu_kernel<3, TS, DT, EPI>(C);
    case 4: return valu_kernel<4, TS, DT, EPI>(C);
    case 5: return valu_kernel<5, TS, DT, EPI>(C);
    case 6: return valu_kernel<6, TS, DT, EPI>(C);
    case 7: return valu_kernel<7, TS, DT, EPI>(C);
    case 8: return valu_kernel<8, TS, DT, EPI>(C);
    default:
      if constexpr (EPI == kEpiFoldAll) return ValuChoice{nullptr, 0, 0};  // B <= 8 only
      // Rows of exactly 256 chunks, one-shot (plain or fused epilogue): A
      // staged through LDS.
      if constexpr (!TS) {
        if (C == 16 * 16)
          return ValuChoice{reinterpret_cast<const void*>(&gemv_ar_mfma_lds<DT, EPI>),
                            (kMfmaLCons + kMfmaLProd) * 64, kMfmaLRows, true, kMfmaLLdsBytes};
      }
      return mfma_x_in_lds(C)
                 ? ValuChoice{reinterpret_cast<const void*>(
                                  &gemv_ar_mfma<kMfmaWaves, 8, TS, DT, EPI>),
                              (kMfmaWaves + 1) * 64, kBigTile}
                 : ValuChoice{reinterpret_cast<const void*>(
                                  &gemv_ar_mfma_xmem<kMfmaWaves, 8, TS, DT, EPI>),
                              (kMfmaWaves + 1) * 64, kBigTile};
  }
}

}  // namespace

size_t gemv_lds_bytes(int W, int B, int C, bool epi, int tile_rows) {
  if (tile_rows == kLongRows) return ((size_t)B * C + 2) * 16;  // x, zero and sink chunks
  // The peer tile, then (with the epilogue) 16 x 16 squares, 16 1/rms and
  // up to 8 waves x 16 partial sums.
  const size_t tail = ((size_t)W * tile_rows * B + 1) * sizeof(float) +
                      (epi ? (size_t)(256 + 16 + 8 * 16) * sizeof(float) : 0);
  const size_t partials = (size_t)kMfmaWaves * kBigTile * 16 * sizeof(float);
  if (B <= 8) return ((size_t)B * C + 2) * 16 + tail;
  if (mfma_x_in_lds(C)) return (size_t)16 * (C + 1) * 16 + partials + tail;
  return partials + tail;
}

bool select_gemv_kernel(int W, int B, int C, int64_t tiles16, bool epi, bool two_shot,
                        bool slot_bf16, bool out_bf16, Launch* out) {
  if (W < 1 || W > GSA_MAX_W || B < 1 || B > GSA_MAX_B || C < 1) return false;
  if (B <= 8 && (size_t)B * C * 16 > GSA_MAX_X_LDS_BYTES) return false;  // x staged in LDS
  if (epi && two_shot) return false;  // separate entry points
  const bool typed = slot_bf16 || out_bf16;
  if (typed && (epi || two_shot)) return false;  // element types: the plain one-shot call only
  const bool fold_all = epi && B <= 8 && C <= 64 && tiles16 * B <= kEpiFoldAllWords;
  const ValuChoice k = two_shot                 ? pick_kernel<true, kDtF32, kEpiNone>(B, C)
                       : fold_all              ? pick_kernel<false, kDtF32, kEpiFoldAll>(B, C)
                       : epi                   ? pick_kernel<false, kDtF32, kEpiFoldOne>(B, C)
                       : slot_bf16 && out_bf16 ? pick_kernel<false, kDtBf16, kEpiNone>(B, C)
                       : typed                 ? pick_kernel<false, kDtMixed, kEpiNone>(B, C)
                                               : pick_kernel<false, kDtF32, kEpiNone>(B, C);
  if (!k.kernel) return false;
  *out = {k.kernel, (unsigned)k.threads,
          k.fixed_lds ? k.lds_bytes : gemv_lds_bytes(W, B, C, epi, k.tile_rows), k.tile_rows};
  return true;
}

hipError_t launch_gemv(const Launch& l, const GemvArgs& a, hipStream_t s) {
  void* args[] = {const_cast<GemvArgs*>(&a)};
  return hipLaunchKernel(l.kernel, dim3((unsigned)a.tiles), dim3(l.block), args, l.lds_bytes, s);
}

hipError_t launch_peer_publish(float* slots, uint32_t* pad, const void* values, int peer,
                               int64_t NB, bool slot_bf16, int row_stride, int64_t nflags,
                               uint32_t epoch, uint64_t delay_ticks, hipStream_t s) {
  hipLaunchKernelGGL(peer_publish_kernel, dim3(1), dim3(256), 0, s, slots, pad, values, peer, NB,
                     slot_bf16 ? 1 : 0, row_stride, nflags, epoch, delay_ticks);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_clear_words(uint32_t* p, int64_t n, hipStream_t s) {
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(clear_words_kernel, dim3(grid), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_pad_reset(uint32_t* pad, int W, int row_stride, int tiles,
                            uint32_t published_mask, float* epi_scratch, hipStream_t s) {
  uint32_t* epi = reinterpret_cast<uint32_t*>(epi_scratch);
  const int64_t epi_words = epi_scratch_words(tiles);
  const int64_t total =
      std::max<int64_t>(GSA_PAD_HEADER_WORDS + 2 * (int64_t)W * row_stride, epi_words);
  const unsigned block = 256;
  const unsigned grid = (unsigned)((total + block - 1) / block);
  hipLaunchKernelGGL(pad_reset_kernel, dim3(grid), dim3(block), 0, s, pad, W, row_stride,
                     published_mask, epi, epi_words);
  return hipGetLastError();
}

}  // namespace gsa
