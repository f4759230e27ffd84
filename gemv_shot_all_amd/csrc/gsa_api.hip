// gsa_api.hip -- host side of libgsa: the C ABI declared in include/gsa.h.
//
// Symmetric buffer = W fp32 slots + signal pad in one device allocation, made
// once at init (the PyTorch Symmetric Memory docs, API reference of empty():
// a host-synchronous allocation meant for initialization, reused afterwards;
// the writing-your-own-kernel section: a signal pad accompanies every
// symmetric allocation).  A registry of live buffers lets every call check
// that the slots/pad pointers belong together and match (W, N, B) in O(1),
// like the constant-time is_symm_mem_tensor() check of the same API.

#include <atomic>
#include <cmath>
#include <mutex>
#include <unordered_map>
#include <unordered_set>

#include "gsa_internal.h"

struct gsa_symm {
  int W;
  int64_t N;
  int B;
  int slot_dtype;   // GSA_DTYPE_F32 or GSA_DTYPE_BF16
  int64_t row_stride;
  int64_t tiles;
  size_t bytes;
  void* base;
  float* slots;
  uint32_t* pad;
  float* gathered;  // the two-shot variant's reduced chunks (N x B fp32)
  float* ssq;       // the fused epilogue's scratch
  int device;
};

// The MoE GEMM + combine all-to-all: W combine buffers and W pads in one
// device allocation.
struct gsa_a2a {
  int W;
  int ne;
  int64_t H;
  int64_t rows_out;
  int64_t row_stride;
  int64_t pad_words;
  void* base;
  float* bufs;
  uint32_t* pads;
  int device;
};

namespace {

std::mutex g_mu;
std::unordered_map<uintptr_t, gsa_symm*> g_by_slots;  // slots -> handle
std::unordered_map<uintptr_t, gsa_symm*> g_by_pad;    // pad -> handle
std::unordered_set<const void*> g_big_lds_ready;      // kernels opted in to > 64 KB LDS
std::atomic<uint32_t> g_timeout_us{100000};
std::unordered_map<int, uint64_t> g_clock_khz;        // device -> wall clock rate

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// Flag tiles of the GEMV pad (4 rows each), 16-row tiles (the fused
// epilogue's records, the two-shot chunks), MoE feature tiles.
int64_t tiles_of(int64_t N) { return (N + GSA_FLAG_TILE_ROWS - 1) / GSA_FLAG_TILE_ROWS; }
int64_t big_tiles_of(int64_t N) {
  return (N + gsa::kBigTileRows - 1) / gsa::kBigTileRows;
}
int64_t moe_tiles_of(int64_t H) { return (H + GSA_MOE_TILE_ROWS - 1) / GSA_MOE_TILE_ROWS; }
int64_t moe_row_stride(int64_t H) { return (int64_t)round_up((size_t)moe_tiles_of(H), 64); }

gsa_symm* find_by_slots(const void* slots) {
  auto it = g_by_slots.find((uintptr_t)slots);
  return it == g_by_slots.end() ? nullptr : it->second;
}
gsa_symm* find_by_pad(const void* pad) {
  auto it = g_by_pad.find((uintptr_t)pad);
  return it == g_by_pad.end() ? nullptr : it->second;
}

// Live handles by address: a handle is never dereferenced before it is found
// here, so a stale or foreign pointer yields GSA_EINVAL, not a fault.
std::unordered_set<const gsa_symm*> g_handles;

bool known(const gsa_symm* h) { return h && g_handles.count(h) != 0; }

std::unordered_set<const gsa_a2a*> g_a2a;                  // live MoE handles
std::unordered_map<uintptr_t, gsa_a2a*> g_a2a_by_pads;     // pads -> handle
bool known(const gsa_a2a* h) { return h && g_a2a.count(h) != 0; }

// Wall-clock ticks for `us` microseconds on the current device.
int ticks_for(uint32_t us, uint64_t* ticks) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GSA_EHIP;
  uint64_t khz;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_clock_khz.find(dev);
    if (it != g_clock_khz.end()) {
      khz = it->second;
    } else {
      int rate = 0;
      if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
          rate <= 0)
        return GSA_EHIP;
      khz = (uint64_t)rate;
      g_clock_khz[dev] = khz;
    }
  }
  *ticks = (uint64_t)us * khz / 1000u + 1u;
  return GSA_OK;
}

}  // namespace

// The entry point that allocates nothing (gsa_gemv_allreduce_rmsnorm_noalloc)
// keeps the fused epilogue's scratch -- one record of partial sums per
// 16-row tile, then the 1/rms copies and the started counts -- in this
// file-scope device array instead of the buffer's own scratch.  Each device
// holds its own copy until the process ends.  Host code never uses the
// array's name as an address: the address comes from hipGetSymbolAddress,
// once per device (g_scratch_ptr), with that device current.
namespace {
constexpr int64_t kNoAllocMaxTiles = 2048;  // 16-row tiles: N <= 32768
constexpr int64_t kNoAllocScratchWords = gsa::epi_scratch_words(kNoAllocMaxTiles);
}  // namespace
static __device__ __align__(256) float scratch[kNoAllocScratchWords];

namespace {
std::unordered_map<int, float*> g_scratch_ptr;  // device -> address of its `scratch`

// The address of this device's `scratch` (looked up on the first call on
// the device).  No allocation.
int scratch_of_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GSA_EHIP;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return GSA_OK;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return GSA_EHIP;
  }
  g_scratch_ptr[dev] = static_cast<float*>(ptr);
  *out = static_cast<float*>(ptr);
  return GSA_OK;
}
}  // namespace

extern "C" {

int64_t gsa_signal_pad_row_stride(int64_t N) {
  if (N < 1) return -1;
  const int64_t groups = (tiles_of(N) + GSA_FLAG_GROUP_TILES - 1) / GSA_FLAG_GROUP_TILES;
  return (int64_t)round_up((size_t)groups * GSA_FLAG_GROUP_WORDS, 64);
}

int gsa_symm_alloc_dtype(int W, int64_t N, int B, int slot_dtype, gsa_symm** out) {
  if (!out || W < 1 || W > GSA_MAX_W || N < 1 || B < 1 || B > GSA_MAX_B) return GSA_EINVAL;
  if (slot_dtype != GSA_DTYPE_F32 && slot_dtype != GSA_DTYPE_BF16) return GSA_EINVAL;
  if (N > ((int64_t)1 << 40)) return GSA_EINVAL;
  *out = nullptr;
  const int64_t stride = gsa_signal_pad_row_stride(N);
  const size_t elem = slot_dtype == GSA_DTYPE_BF16 ? sizeof(uint16_t) : sizeof(float);
  const size_t slot_bytes = round_up((size_t)W * (size_t)N * (size_t)B * elem, kAlign);
  const size_t pad_words = GSA_PAD_HEADER_WORDS + 2 * (size_t)W * (size_t)stride;
  const size_t gathered_bytes = round_up((size_t)N * (size_t)B * sizeof(float), kAlign);
  const size_t pad_bytes = round_up(pad_words * sizeof(uint32_t), kAlign);
  // The epilogue's scratch: one record per 16-row tile, then the 1/rms copies and
  // the started counts.
  const size_t ssq_bytes =
      round_up((size_t)gsa::epi_scratch_words(big_tiles_of(N)) * sizeof(float), kAlign);
  const size_t bytes = slot_bytes + pad_bytes + gathered_bytes + ssq_bytes;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GSA_EHIP;
  void* base = nullptr;
  if (hipMalloc(&base, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return GSA_ENOMEM;
  }
  uint32_t* pad = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + slot_bytes);
  uint32_t hdr[GSA_PAD_HEADER_WORDS] = {0};
  hdr[gsa::kHdrTimeoutKey] = 0xFFFFFFFFu;
  hdr[gsa::kHdrStateTile] = 0xFFFFFFFFu;
  hdr[gsa::kHdrEpiWaitTile] = 0xFFFFFFFFu;
  if (hipMemset(base, 0, bytes) != hipSuccess ||
      hipMemcpy(pad, hdr, sizeof hdr, hipMemcpyHostToDevice) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(base);
    return GSA_EHIP;
  }
  float* gathered = reinterpret_cast<float*>(static_cast<char*>(base) + slot_bytes + pad_bytes);
  float* ssq = reinterpret_cast<float*>(static_cast<char*>(base) + slot_bytes + pad_bytes +
                                        gathered_bytes);
  gsa_symm* h = new gsa_symm{W, N, B, slot_dtype, stride, big_tiles_of(N), bytes, base,
                             static_cast<float*>(base), pad, gathered, ssq, dev};
  std::lock_guard<std::mutex> lk(g_mu);
  g_by_slots[(uintptr_t)h->slots] = h;
  g_by_pad[(uintptr_t)h->pad] = h;
  g_handles.insert(h);
  *out = h;
  return GSA_OK;
}

int gsa_symm_alloc(int W, int64_t N, int B, gsa_symm** out) {
  return gsa_symm_alloc_dtype(W, N, B, GSA_DTYPE_F32, out);
}

int gsa_symm_free(gsa_symm* h) {
  if (!h) return GSA_OK;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!known(h)) return GSA_EINVAL;
    g_by_slots.erase((uintptr_t)h->slots);
    g_by_pad.erase((uintptr_t)h->pad);
    g_handles.erase(h);
  }
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e == hipSuccess && prev != h->device) e = hipSetDevice(h->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipFree(h->base);
  if (prev != h->device) (void)hipSetDevice(prev);
  delete h;
  return e == hipSuccess ? GSA_OK : GSA_EHIP;
}

float* gsa_symm_slots(const gsa_symm* h) {
  std::lock_guard<std::mutex> lk(g_mu);
  return known(h) ? h->slots : nullptr;
}

uint32_t* gsa_symm_signal_pad(const gsa_symm* h) {
  std::lock_guard<std::mutex> lk(g_mu);
  return known(h) ? h->pad : nullptr;
}

float* gsa_symm_gathered(const gsa_symm* h) {
  std::lock_guard<std::mutex> lk(g_mu);
  return known(h) ? h->gathered : nullptr;
}

int gsa_signal_pad_reset(uint32_t* pad, int W, int64_t N, uint32_t published_mask,
                         void* stream) {
  if (!pad || W < 1 || W > GSA_MAX_W || N < 1) return GSA_EINVAL;
  if (published_mask >> W) return GSA_EINVAL;
  int64_t stride, tiles;
  float* epi_scratch;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    gsa_symm* h = find_by_pad(pad);
    if (!h || h->W != W || h->N != N) return GSA_EINVAL;
    stride = h->row_stride;
    tiles = h->tiles;
    epi_scratch = h->ssq;
  }
  hipError_t e = gsa::launch_pad_reset(pad, W, (int)stride, (int)tiles, published_mask,
                                       epi_scratch, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GSA_OK : GSA_EHIP;
}

}  // extern "C"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Every GEMV entry point: validate, fill the launch arguments, enqueue one
// kernel.  out_dtype is the element type of out; bf16_slots_ok whether the
// entry point accepts a buffer whose slots are bf16 (the plain one-shot call
// with element types only; the others take fp32 slots).
// epi_scratch: the epilogue's scratch to use instead of the buffer's own
// (the no-allocation entry point); its counts and 1/rms copies are cleared
// by a small kernel ahead of the call.
int enqueue_call(const uint16_t* A_r, const uint16_t* x, void* slots_any, uint32_t* pad,
                 float* gathered, void* out_any, int out_dtype, bool bf16_slots_ok, int W,
                 int rank, int64_t N, int64_t K, int B, const gsa_epilogue* ep, void* stream,
                 float* epi_scratch = nullptr) {
  float* slots = static_cast<float*>(slots_any);
  float* out = static_cast<float*>(out_any);
  if (out_dtype != GSA_DTYPE_F32 && out_dtype != GSA_DTYPE_BF16) return GSA_EINVAL;
  // Scalars first: these checks touch no HIP state.
  if (W < 1 || W > GSA_MAX_W || rank < 0 || rank >= W) return GSA_EINVAL;
  if (N < 1 || B < 1 || B > GSA_MAX_B || K < 1 || K % W != 0) return GSA_EINVAL;
  const int64_t Ks = K / W;
  if (Ks % 8 != 0 || Ks / 8 > (1 << 20)) return GSA_EINVAL;
  if (tiles_of(N) > 0x7FFFFFFF / 8) return GSA_EINVAL;
  if (!A_r || !x || !slots || !pad || !out) return GSA_EINVAL;
  if (!aligned16(A_r) || !aligned16(x) || !aligned16(slots) || !aligned16(pad) ||
      !aligned16(out))
    return GSA_EINVAL;
  // A_r is addressed through a 32-bit buffer resource.
  if (N > ((int64_t)0x7FFFFFF0 / 2) / Ks) return GSA_EINVAL;
  if (ep) {
    if (!ep->y || (ep->y_dtype != GSA_DTYPE_F32 && ep->y_dtype != GSA_DTYPE_BF16))
      return GSA_EINVAL;
    if (!aligned(ep->y, ep->y_dtype == GSA_DTYPE_F32 ? 4 : 2)) return GSA_EINVAL;
    if ((ep->bias && !aligned(ep->bias, 4)) || (ep->rms_weight && !aligned(ep->rms_weight, 4)) ||
        (ep->inv_rms && !aligned(ep->inv_rms, 4)))
      return GSA_EINVAL;
    if (!std::isfinite(ep->eps) || ep->eps < 0.0f) return GSA_EINVAL;
    if (N > ((int64_t)1 << 24)) return GSA_EINVAL;  // N is exact as a float divisor
  }
  const int C = (int)(Ks / 8);
  gsa::Launch l;
  gsa::GemvArgs a;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    gsa_symm* h = find_by_slots(slots);
    if (!h || h->pad != pad || h->W != W || h->N != N || h->B != B) return GSA_EINVAL;
    if (h->slot_dtype == GSA_DTYPE_BF16 && !bf16_slots_ok) return GSA_EINVAL;
    a.slot_bf16 = h->slot_dtype == GSA_DTYPE_BF16 ? 1 : 0;
    if (gathered && h->gathered != gathered) return GSA_EINVAL;
    // kernel instances with the element types fixed (both fp32 or both
    // bf16), or tested at run time (mixed)
    if (!gsa::select_gemv_kernel(W, B, C, h->tiles, ep != nullptr, gathered != nullptr,
                                 a.slot_bf16 != 0, out_dtype == GSA_DTYPE_BF16, &l))
      return GSA_EINVAL;
    a.row_stride = (int)h->row_stride;
    a.tiles = (int)((N + l.tile_rows - 1) / l.tile_rows);
    a.epi_tiles = (int)h->tiles;  // 16-row tiles, whatever the kernel's tile
    a.ssq = h->ssq;
    if (l.lds_bytes > 65536 && !g_big_lds_ready.count(l.kernel)) {
      // Opt in once to the largest dynamic LDS any shape of this kernel may use.
      if (hipFuncSetAttribute(l.kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GSA_MAX_X_LDS_BYTES + 16384) != hipSuccess) {
        (void)hipGetLastError();
      }
      g_big_lds_ready.insert(l.kernel);
    }
  }
  a.A = A_r;
  a.x = x;
  a.slots = slots;
  a.pad = pad;
  a.out = out;
  a.out_bf16 = out_dtype == GSA_DTYPE_BF16 ? 1 : 0;
  a.N = N;
  a.C = C;
  a.B = B;
  a.W = W;
  a.rank = rank;
  a.gathered = gathered;
  a.chunk_tiles = (int)big_tiles_of((N + W - 1) / W);  // whole 16-row tiles per rank
  a.epi = ep ? 1 : 0;
  a.y_bf16 = ep && ep->y_dtype == GSA_DTYPE_BF16 ? 1 : 0;
  a.eps = ep ? ep->eps : 0.0f;
  a.bias = ep ? ep->bias : nullptr;
  a.rms_w = ep ? ep->rms_weight : nullptr;
  a.y = ep ? ep->y : nullptr;
  a.inv_rms = ep ? ep->inv_rms : nullptr;
  int rc = ticks_for(g_timeout_us.load(std::memory_order_relaxed), &a.timeout_ticks);
  if (rc != GSA_OK) return rc;
  hipError_t e = hipSuccess;
  if (epi_scratch) {
    // The shared scratch starts cleared for every call (the buffer's own
    // scratch counts calls instead, so its records and 1/rms copies carry
    // each call's mark): the counts, the records and the copies, so that no
    // word a previous call left can pass for one of this call.
    a.ssq = epi_scratch;
    e = gsa::launch_clear_words(reinterpret_cast<uint32_t*>(epi_scratch),
                                gsa::epi_scratch_words(a.epi_tiles), static_cast<hipStream_t>(stream));
  }
  if (e == hipSuccess) e = gsa::launch_gemv(l, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return GSA_EHIP;
  }
  return GSA_OK;
}

}  // namespace

extern "C" {

int gsa_gemv_allreduce(const uint16_t* A_r, const uint16_t* x, float* slots, uint32_t* pad,
                       float* out, int W, int rank, int64_t N, int64_t K, int B, void* stream) {
  return enqueue_call(A_r, x, slots, pad, nullptr, out, GSA_DTYPE_F32, false, W, rank, N, K, B,
                      nullptr, stream);
}

int gsa_gemv_allreduce_dtype(const uint16_t* A_r, const uint16_t* x, void* slots, uint32_t* pad,
                             void* out, int out_dtype, int W, int rank, int64_t N, int64_t K,
                             int B, void* stream) {
  return enqueue_call(A_r, x, slots, pad, nullptr, out, out_dtype, true, W, rank, N, K, B,
                      nullptr, stream);
}

int gsa_gemv_allreduce_two_shot(const uint16_t* A_r, const uint16_t* x, float* slots,
                                uint32_t* pad, float* gathered, float* out, int W, int rank,
                                int64_t N, int64_t K, int B, void* stream) {
  if (!gathered || !aligned16(gathered)) return GSA_EINVAL;
  return enqueue_call(A_r, x, slots, pad, gathered, out, GSA_DTYPE_F32, false, W, rank, N, K, B,
                      nullptr, stream);
}

int gsa_gemv_allreduce_rmsnorm(const uint16_t* A_r, const uint16_t* x, float* slots,
                               uint32_t* pad, float* out, int W, int rank, int64_t N, int64_t K,
                               int B, const gsa_epilogue* ep, void* stream) {
  if (!ep) return GSA_EINVAL;
  return enqueue_call(A_r, x, slots, pad, nullptr, out, GSA_DTYPE_F32, false, W, rank, N, K, B,
                      ep, stream);
}

int gsa_bias_rmsnorm(const float* out, int64_t N, int B, const gsa_epilogue* ep, void* stream) {
  if (!out || !ep || !ep->y || N < 1 || N > ((int64_t)1 << 24) || B < 1 || B > GSA_MAX_B)
    return GSA_EINVAL;
  if (ep->y_dtype != GSA_DTYPE_F32 && ep->y_dtype != GSA_DTYPE_BF16) return GSA_EINVAL;
  if (!aligned(out, 4) || !aligned(ep->y, ep->y_dtype == GSA_DTYPE_F32 ? 4 : 2)) return GSA_EINVAL;
  if ((ep->bias && !aligned(ep->bias, 4)) || (ep->rms_weight && !aligned(ep->rms_weight, 4)) ||
      (ep->inv_rms && !aligned(ep->inv_rms, 4)))
    return GSA_EINVAL;
  if (!std::isfinite(ep->eps) || ep->eps < 0.0f) return GSA_EINVAL;
  if (gsa::launch_bias_rmsnorm(out, N, B, ep->bias, ep->rms_weight, ep->eps, ep->y,
                               ep->y_dtype == GSA_DTYPE_BF16, ep->inv_rms,
                               static_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipGetLastError();
    return GSA_EHIP;
  }
  return GSA_OK;
}

int gsa_peer_publish(void* slots, uint32_t* pad, const void* values, int W, int peer, int64_t N,
                     int B, uint32_t epoch, uint32_t delay_us, void* stream) {
  if (!slots || !pad || !values || W < 1 || W > GSA_MAX_W || peer < 0 || peer >= W || N < 1 ||
      B < 1 || B > GSA_MAX_B || delay_us > 1000000u)
    return GSA_EINVAL;
  bool bf16;
  int64_t stride;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    gsa_symm* h = find_by_slots(slots);
    if (!h || h->pad != pad || h->W != W || h->N != N || h->B != B) return GSA_EINVAL;
    bf16 = h->slot_dtype == GSA_DTYPE_BF16;
    stride = h->row_stride;
  }
  if (((uintptr_t)values & (bf16 ? 1u : 3u)) != 0) return GSA_EINVAL;
  uint64_t ticks = 0;
  if (delay_us > 0) {
    const int rc = ticks_for(delay_us, &ticks);
    if (rc != GSA_OK) return rc;
  }
  const hipError_t e = gsa::launch_peer_publish(
      static_cast<float*>(slots), pad, values, peer, N * (int64_t)B, bf16, (int)stride,
      tiles_of(N), epoch, ticks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return GSA_EHIP;
  }
  return GSA_OK;
}

int gsa_gemv_allreduce_rmsnorm_noalloc(const uint16_t* A_r, const uint16_t* x, float* slots,
                                       uint32_t* pad, float* out, int W, int rank, int64_t N,
                                       int64_t K, int B, const gsa_epilogue* ep, void* stream) {
  if (!ep) return GSA_EINVAL;
  // The epilogue's 16-row tiles must fit the static scratch.
  if (N < 1 || big_tiles_of(N) > kNoAllocMaxTiles) return GSA_EINVAL;
  float* sc = nullptr;
  const int rc = scratch_of_current_device(&sc);
  if (rc != GSA_OK) return rc;
  return enqueue_call(A_r, x, slots, pad, nullptr, out, GSA_DTYPE_F32, false, W, rank, N, K, B,
                      ep, stream, sc);
}

int gsa_signal_pad_status(const uint32_t* pad, void* stream, int* code, int64_t* tile,
                          int* peer) {
  if (!pad || !code || !tile || !peer) return GSA_EINVAL;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!find_by_pad(pad)) return GSA_EINVAL;
  }
  uint32_t hdr[GSA_PAD_HEADER_WORDS];
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(hdr, pad, sizeof hdr, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return GSA_EHIP;
  const uint32_t bits = hdr[gsa::kHdrErrorBits];
  *code = (bits & gsa::kErrState) ? GSA_ESTATE
          : (bits & (gsa::kErrTimeout | gsa::kErrEpiWait)) ? GSA_ETIMEOUT
                                                          : GSA_OK;
  const uint32_t key = hdr[gsa::kHdrTimeoutKey];
  *tile = -1;
  *peer = -1;
  if (bits & gsa::kErrState) {
    *tile = (int64_t)hdr[gsa::kHdrStateTile];
  } else if (key != 0xFFFFFFFFu) {
    *tile = (int64_t)(key / 8u);
    *peer = (int)(key % 8u);
  } else if (bits & gsa::kErrEpiWait) {
    *tile = (int64_t)hdr[gsa::kHdrEpiWaitTile];
  }
  return GSA_OK;
}

int gsa_set_wait_timeout_us(uint32_t us) {
  if (us == 0) return GSA_EINVAL;
  g_timeout_us.store(us, std::memory_order_relaxed);
  return GSA_OK;
}

int64_t gsa_a2a_pad_words(int W, int ne, int64_t H) {
  if (W < 1 || W > GSA_MAX_W || ne < 1 || ne > 256 || H < 1 || H > ((int64_t)1 << 30)) return -1;
  return GSA_PAD_HEADER_WORDS + (int64_t)W * ne * moe_row_stride(H);
}

int gsa_a2a_alloc(int W, int ne, int64_t H, int64_t rows_out, gsa_a2a** out) {
  if (!out) return GSA_EINVAL;
  *out = nullptr;
  const int64_t pad_words = gsa_a2a_pad_words(W, ne, H);
  if (pad_words < 0 || rows_out < 1) return GSA_EINVAL;
  if ((int64_t)W * rows_out > ((int64_t)1 << 40) / H) return GSA_EINVAL;
  const size_t buf_bytes = round_up((size_t)W * rows_out * H * sizeof(float), kAlign);
  const size_t pad_bytes = round_up((size_t)W * pad_words * sizeof(uint32_t), kAlign);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GSA_EHIP;
  void* base = nullptr;
  if (hipMalloc(&base, buf_bytes + pad_bytes) != hipSuccess) {
    (void)hipGetLastError();
    return GSA_ENOMEM;
  }
  if (hipMemset(base, 0, buf_bytes + pad_bytes) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(base);
    return GSA_EHIP;
  }
  uint32_t* pads = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + buf_bytes);
  gsa_a2a* h = new gsa_a2a{W, ne, H, rows_out, moe_row_stride(H), pad_words, base,
                           static_cast<float*>(base), pads, dev};
  std::lock_guard<std::mutex> lk(g_mu);
  g_a2a.insert(h);
  g_a2a_by_pads[(uintptr_t)pads] = h;
  *out = h;
  return GSA_OK;
}

int gsa_a2a_free(gsa_a2a* h) {
  if (!h) return GSA_OK;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!known(h)) return GSA_EINVAL;
    g_a2a_by_pads.erase((uintptr_t)h->pads);
    g_a2a.erase(h);
  }
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e == hipSuccess && prev != h->device) e = hipSetDevice(h->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipFree(h->base);
  if (prev != h->device) (void)hipSetDevice(prev);
  delete h;
  return e == hipSuccess ? GSA_OK : GSA_EHIP;
}

float* gsa_a2a_buffers(const gsa_a2a* h) {
  std::lock_guard<std::mutex> lk(g_mu);
  return known(h) ? h->bufs : nullptr;
}

uint32_t* gsa_a2a_signal_pads(const gsa_a2a* h) {
  std::lock_guard<std::mutex> lk(g_mu);
  return known(h) ? h->pads : nullptr;
}

int gsa_a2a_reset(uint32_t* pads, int W, int ne, int64_t H, uint32_t published_mask,
                  void* stream) {
  if (!pads || W < 1 || W > GSA_MAX_W || (published_mask >> W)) return GSA_EINVAL;
  int64_t stride, pad_words;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_a2a_by_pads.find((uintptr_t)pads);
    if (it == g_a2a_by_pads.end()) return GSA_EINVAL;
    const gsa_a2a* h = it->second;
    if (h->W != W || h->ne != ne || h->H != H) return GSA_EINVAL;
    stride = h->row_stride;
    pad_words = h->pad_words;
  }
  hipError_t e = gsa::launch_a2a_reset(pads, W, ne, (int)stride, pad_words, published_mask,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GSA_OK : GSA_EHIP;
}

int gsa_moe_gemm_all_to_all(const uint16_t* X, const uint16_t* Wd, const int32_t* splits,
                            const int32_t* dst_off, float* bufs, uint32_t* pads, int W,
                            int rank, int ne, int64_t H, int64_t F, int64_t rows_in,
                            int64_t rows_out, void* stream) {
  // Scalars first: these checks touch no HIP state.
  if (W < 1 || W > GSA_MAX_W || rank < 0 || rank >= W || ne < 1 || ne > 256) return GSA_EINVAL;
  if (H < 1 || F < 8 || F % 8 != 0 || F > GSA_MOE_MAX_F || rows_in < 1 || rows_out < 1)
    return GSA_EINVAL;
  if (H * F * 2 >= ((int64_t)1 << 31)) return GSA_EINVAL;  // one expert through a buffer resource
  if (rows_in > ((int64_t)1 << 40) / F) return GSA_EINVAL;
  if (!X || !Wd || !splits || !dst_off || !bufs || !pads) return GSA_EINVAL;
  if (!aligned16(X) || !aligned16(Wd) || !aligned16(bufs) || !aligned16(pads) ||
      ((uintptr_t)splits & 3u) || ((uintptr_t)dst_off & 3u))
    return GSA_EINVAL;
  gsa::MoeArgs a;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_a2a_by_pads.find((uintptr_t)pads);
    if (it == g_a2a_by_pads.end()) return GSA_EINVAL;
    const gsa_a2a* h = it->second;
    if (h->bufs != bufs || h->W != W || h->ne != ne || h->H != H || h->rows_out != rows_out)
      return GSA_EINVAL;
    a.row_stride = (int)h->row_stride;
    a.pad_words = h->pad_words;
  }
  a.X = X;
  a.Wd = Wd;
  a.splits = splits;
  a.dst_off = dst_off;
  a.bufs = bufs;
  a.pads = pads;
  a.W = W;
  a.rank = rank;
  a.ne = ne;
  a.C = (int)(F / 8);
  a.tiles = (int)moe_tiles_of(H);
  a.H = H;
  a.F = F;
  a.rows_in = rows_in;
  a.rows_out = rows_out;
  int rc = ticks_for(g_timeout_us.load(std::memory_order_relaxed), &a.timeout_ticks);
  if (rc != GSA_OK) return rc;
  hipError_t e = gsa::launch_moe(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return GSA_EHIP;
  }
  return GSA_OK;
}

int gsa_a2a_status(const uint32_t* pads, int rank, void* stream, int* code, int64_t* tile,
                   int* peer) {
  if (!pads || !code || !tile || !peer) return GSA_EINVAL;
  int64_t pad_words;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_a2a_by_pads.find((uintptr_t)pads);
    if (it == g_a2a_by_pads.end() || rank < 0 || rank >= it->second->W) return GSA_EINVAL;
    pad_words = it->second->pad_words;
  }
  uint32_t hdr[GSA_PAD_HEADER_WORDS];
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(hdr, pads + (int64_t)rank * pad_words, sizeof hdr, hipMemcpyDeviceToHost,
                     s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return GSA_EHIP;
  const uint32_t bits = hdr[gsa::kHdrErrorBits];
  *tile = -1;
  *peer = -1;
  if (bits & gsa::kErrSplit) {
    *code = GSA_ESPLIT;
    *tile = (int64_t)hdr[gsa::kHdrSplitExpert];
  } else if (bits & gsa::kErrState) {
    *code = GSA_ESTATE;
    *tile = (int64_t)hdr[gsa::kHdrStateTile];
  } else if (bits & gsa::kErrTimeout) {
    *code = GSA_ETIMEOUT;
    const uint32_t key = hdr[gsa::kHdrTimeoutKey];
    *tile = (int64_t)(key / 8u);
    *peer = (int)(key % 8u);
  } else {
    *code = GSA_OK;
  }
  return GSA_OK;
}

const char* gsa_strerror(int code) {
  switch (code) {
    case GSA_OK: return "ok";
    case GSA_EINVAL: return "invalid argument";
    case GSA_ENOMEM: return "device allocation failed";
    case GSA_EHIP: return "HIP runtime error";
    case GSA_ETIMEOUT: return "signal-pad wait timed out";
    case GSA_ESTATE: return "own flag row not usable (marked published or epochs exhausted)";
    case GSA_ESPLIT: return "a split or offset on the device is out of range, or an expert got "
                            "more tokens than it takes";
    default: return "unknown error";
  }
}

}  // extern "C"
