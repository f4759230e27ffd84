// gsa_internal.h -- declarations shared by the host side and the kernels of
// libgsa.  Not part of the public ABI (that is include/gsa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gsa.h"

namespace gsa {

// Status words at the head of the signal pad.
enum : int {
  kHdrErrorBits = 0,   // atomicOr: kErrTimeout | kErrState
  kHdrTimeoutKey = 1,  // atomicMin of tile * 8 + peer, 0xFFFFFFFF = none
  kHdrStateTile = 2,   // atomicMin of the tile with a bad own flag row
  kHdrEpiWaitTile = 6, // atomicMin of a tile whose epilogue wait expired, 0xFFFFFFFF = none
  kHdrSplitExpert = 7, // MoE: atomicMin of a local expert with a bad split table
};
// The epilogue's scratch (fp32 / uint32 words, 128-byte lines of 32 words):
//   records   tiles lines: 16 64-bit words, column c = (tag << 32) | bits of
//             the tile's sum of squares (tag: the call's mark, top bit set if
//             the tile left its rows to the reducing workgroup)
//   inv       kEpiGroups lines: 16 64-bit words, column c = (mark << 32) | bits of 1/rms
//   started   kEpiGroups lines: a 64-bit count at word 0
// Tile t belongs to group t % kEpiGroups; spreading the counts and the 1/rms
// copies over separate lines keeps the tiles' atomics and polls from queueing
// on one address.  The pad reset clears all of it.
constexpr int kEpiRecordWords = 32;
constexpr int kEpiGroups = 64;
__host__ __device__ constexpr int64_t epi_inv_off(int64_t tiles) { return tiles * kEpiRecordWords; }
__host__ __device__ constexpr int64_t epi_started_off(int64_t tiles) {
  return epi_inv_off(tiles) + kEpiGroups * kEpiRecordWords;
}
__host__ __device__ constexpr int64_t epi_scratch_words(int64_t tiles) {
  return epi_started_off(tiles) + kEpiGroups * kEpiRecordWords;
}
enum : uint32_t { kErrTimeout = 1u, kErrState = 2u, kErrEpiWait = 4u, kErrSplit = 8u };

// Everything one launch needs.  Built on the host per call, passed by value.
struct GemvArgs {
  const uint16_t* A;      // N x Ks bf16 bits
  const uint16_t* x;      // B x Ks bf16 bits
  float* slots;           // W x N x B fp32, or bf16 bits if slot_bf16
  uint32_t* pad;          // header + W flag rows
  float* out;             // N x B fp32, or bf16 bits if out_bf16
  int slot_bf16;          // the slots hold bf16 values (published y rounded to bf16)
  int out_bf16;           // out is bf16 (the fp32 sum rounded to nearest, ties to even)
  int64_t N;
  int C;                  // 16-byte chunks per row = Ks / 8
  int B;
  int W;
  int rank;
  int row_stride;         // words between flag rows
  int tiles;              // workgroup tiles: ceil(N / tile rows of the kernel)
  int epi_tiles;          // the fused epilogue's 16-row tiles: ceil(N / 16)
  uint64_t timeout_ticks; // device wall-clock ticks a wait may take
  // Two-shot variant (the kernels' TS instances): rank p owns the 16-row
  // blocks [p * chunk_tiles, (p + 1) * chunk_tiles), reduces them into gathered
  // (N x B) and raises its reduced-chunk flag (pad row W + p); other rows are
  // copied from their owner's gathered rows once its flag shows the epoch.
  int chunk_tiles;
  float* gathered;
  // Fused epilogue (bias, RMSNorm over rows, y in fp32 or bf16); epi == 0:
  // none, and the fields below are unused.
  int epi;
  int y_bf16;
  float eps;
  const float* bias;      // N fp32 or null
  const float* rms_w;     // N fp32 or null
  void* y;                // N x B
  float* inv_rms;         // B fp32 or null
  float* ssq;             // the epilogue's scratch (records, 1/rms copies, started counts)
};

// Rows per flag tile of the pad (GSA_FLAG_TILE_ROWS) and per workgroup of the
// kernels that run the fused epilogue, the two-shot variant and MFMA.
constexpr int kBigTileRows = 16;

// A ready-to-launch kernel choice for one (B, C) shape.
struct Launch {
  const void* kernel;
  unsigned block;         // threads per workgroup
  size_t lds_bytes;       // dynamic LDS
  int tile_rows;          // output rows per workgroup (4 or 16)
};

// Pick the kernel for W ranks, batch B (1..16) and C chunks per row (with
// the epilogue's extra LDS if epi).  Returns false if the shape exceeds the
// LDS staging bound.
// The fused epilogue's bias + RMSNorm as a kernel of its own, over an out
// already written (B workgroups).
hipError_t launch_bias_rmsnorm(const float* out, int64_t N, int B, const float* bias,
                               const float* w, float eps, void* y, bool y_bf16, float* inv_rms,
                               hipStream_t s);

// tiles16: the call's 16-row tiles (the epilogue's record count).
bool select_gemv_kernel(int W, int B, int C, int64_t tiles16, bool epi, bool two_shot,
                        bool slot_bf16, bool out_bf16, Launch* out);
// Dynamic LDS bytes a kernel of tile_rows rows per workgroup needs for (W, B, C, epi).
size_t gemv_lds_bytes(int W, int B, int C, bool epi, int tile_rows);

hipError_t launch_gemv(const Launch& l, const GemvArgs& a, hipStream_t s);
// Zero n words at p with a small kernel (graph-capturable, unlike a memset node).
hipError_t launch_clear_words(uint32_t* p, int64_t n, hipStream_t s);
// The one-GPU stand-in for a peer's push (see gsa_peer_publish).
hipError_t launch_peer_publish(float* slots, uint32_t* pad, const void* values, int peer,
                               int64_t NB, bool slot_bf16, int row_stride, int64_t nflags,
                               uint32_t epoch, uint64_t delay_ticks, hipStream_t s);
// Also clears the fused epilogue's scratch after its records (flags and
// counts), so the next call starts counting from zero.
hipError_t launch_pad_reset(uint32_t* pad, int W, int row_stride, int tiles,
                            uint32_t published_mask, float* epi_scratch, hipStream_t s);

// The MoE GEMM + combine all-to-all (moe_a2a.hip).
struct MoeArgs {
  const uint16_t* X;        // rows_in x F bf16 bits
  const uint16_t* Wd;       // ne x H x F bf16 bits
  const int32_t* splits;    // 2 x ne x W: lengths, then offsets in X
  const int32_t* dst_off;   // W x ne
  float* bufs;              // W x rows_out x H fp32
  uint32_t* pads;           // W pads of pad_words words
  int W, rank, ne;
  int C;                    // F / 8 (16-byte chunks per row)
  int tiles;                // ceil(H / 16)
  int row_stride;           // words between flag rows
  int64_t H, F, rows_in, rows_out, pad_words;
  uint64_t timeout_ticks;
};
hipError_t launch_moe(const MoeArgs& a, hipStream_t s);
hipError_t launch_a2a_reset(uint32_t* pads, int W, int ne, int row_stride, int64_t pad_words,
                            uint32_t published_mask, hipStream_t s);

}  // namespace gsa
