// C ABI of libonebit.so (declared in include/onebit.h): argument checks,
// the tensor-table descriptor, workspace layout and kernel launches.  All
// arithmetic runs in the kernels of onebit_kernels.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>
#include <vector>

#include "onebit.h"
#include "onebit_host.hpp"
#include "onebit_kernels.hpp"
#include "onebit_big.hpp"

using namespace onebit;

static_assert(onebit::kMaxWorkers == onebit_host::kMaxWorkers, "one worker bound");

struct onebit_layer_table {
  int32_t L = 0;
  int32_t chunk = 0;
  int64_t N = 0;
  int64_t K = 0;
  int64_t S = 0;  // (chunk, tensor) segments
  int device = -1;  // the device that holds dblock
  int cus = 0;      // its compute units (sizes the persistent pass-A grid)
  int64_t max_tseg = 0;  // segments of the tensor that has the most
  void* dblock = nullptr;
  DevTable dev{};
};

namespace {

using onebit_host::aligned16;
using onebit_host::aligned4;
using onebit_host::Bytes;
using onebit_host::check_hparams;
using onebit_host::check_n;
using onebit_host::check_W;
using onebit_host::chunk_supported;
using onebit_host::fail;
using onebit_host::ok;
using onebit_host::Spans;

// Checks a device array pointer argument.
#define CHECK_PTR(p, name)                                                                   \
  do {                                                                                       \
    if (!(p)) return fail(ONEBIT_EINVAL, "%s: %s is NULL", __func__, name);                  \
    if (!aligned16(p)) return fail(ONEBIT_EALIGN, "%s: %s is not 16-byte aligned", __func__, \
                                   name);                                                    \
  } while (0)

// Sign-word and scale arrays are read and written one 32-bit word at a time.
#define CHECK_WORDS(p, name)                                                                 \
  do {                                                                                       \
    if (!(p)) return fail(ONEBIT_EINVAL, "%s: %s is NULL", __func__, name);                  \
    if (!aligned4(p)) return fail(ONEBIT_EALIGN, "%s: %s is not 4-byte aligned", __func__,   \
                                  name);                                                     \
  } while (0)

// The optional status word takes 32-bit atomics.
#define CHECK_OPT_WORDS(p, name)                                                             \
  do {                                                                                       \
    if ((p) && !aligned4(p))                                                                 \
      return fail(ONEBIT_EALIGN, "%s: %s is not 4-byte aligned", __func__, name);            \
  } while (0)

#define CHECK_OPT_PTR(p, name)                                                               \
  do {                                                                                       \
    if ((p) && !aligned16(p))                                                                \
      return fail(ONEBIT_EALIGN, "%s: %s is not 16-byte aligned", __func__, name);           \
  } while (0)

int launch_status(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ONEBIT_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

Coef make_coef(const onebit_hparams& h) {
  Coef c;
  c.beta1 = h.beta1;
  c.beta2 = h.beta2;
  c.eta = h.eta;
  c.lr = h.lr;
  c.a1 = 1.0f - h.beta1;
  c.a2 = 1.0f - h.beta2;
  c.kp = 1.0f + h.kappa;
  c.km = 1.0f - h.kappa;
  c.c_min = h.c_min;
  c.c_max = h.c_max;
  c.f_min = h.f_min;
  c.f_max = h.f_max;
  c.wd = h.weight_decay;
  c.bias = h.bias_step >= 1 ? 1 : 0;
  // 1 - beta^t in double from the fp32 beta, rounded once
  c.bc1 = c.bias ? (float)(1.0 - std::pow((double)h.beta1, (double)h.bias_step)) : 1.0f;
  c.bc2 = c.bias ? (float)(1.0 - std::pow((double)h.beta2, (double)h.bias_step)) : 1.0f;
  c.cd = h.c_avg_decay;
  c.cd1 = 1.0f - h.c_avg_decay;
  return c;
}

// A table's device block lives on one device; a call made with another
// device current would hand its kernels a foreign address.
int check_table(const onebit_layer_table* t, const char* fn) {
  if (!t || !t->dblock) return fail(ONEBIT_EINVAL, "%s: table is NULL", fn);
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ONEBIT_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev != t->device)
    return fail(ONEBIT_EINVAL, "%s: table was created on device %d, current device is %d", fn,
                t->device, dev);
  return ONEBIT_OK;
}

// Device views of the workspace (layout in onebit_host::ws_offsets).
struct Ws {
  double* seg_x;
  double* seg_u;
  float* seg_max;
  float* c_layer;
};

size_t ws_bytes(const onebit_layer_table* t) { return onebit_host::ws_bytes(t->S, t->L); }

Ws ws_view(const onebit_layer_table* t, void* ws) {
  char* p = static_cast<char*>(ws);
  const onebit_host::WsOffsets o = onebit_host::ws_offsets(t->S);
  Ws w;
  w.seg_x = reinterpret_cast<double*>(p + o.seg_x);
  w.seg_u = reinterpret_cast<double*>(p + o.seg_u);
  w.seg_max = reinterpret_cast<float*>(p + o.seg_max);
  w.c_layer = reinterpret_cast<float*>(p + o.c_layer);
  return w;
}

// Dispatch a chunk-templated launch on the runtime chunk size.
template <template <int> class F, typename... A>
void by_chunk(int32_t chunk, A&&... a) {
  switch (chunk) {
    case 64: F<64>::run(a...); break;
    case 128: F<128>::run(a...); break;
    case 256: F<256>::run(a...); break;
    case 512: F<512>::run(a...); break;
    case 1024: F<1024>::run(a...); break;
    case 2048: F<2048>::run(a...); break;
    case 4096: F<4096>::run(a...); break;
    case 8192: F<8192>::run(a...); break;
    case 16384: F<16384>::run(a...); break;
    default: break;
  }
}

// Launch k with one workgroup of Geo<C>::T threads (C/16, and 64 for chunks
// shorter than 1024) per chunk of an n-element buffer; k takes the number
// of full chunks first (block 0 takes the partial last chunk, if any).
template <int C, typename KF, typename... A>
void launch_chunks(int64_t n, hipStream_t st, KF k, A... args) {
  const int64_t K = (n + C - 1) / C;
  if (K > 0) hipLaunchKernelGGL(k, dim3((unsigned)K), dim3(Geo<C>::T), 0, st, n / C, args...);
}

// The same for a kernel laid out with SPT float4 slots per thread
// (Geo<C, SPT>::T threads per chunk).
template <int C, int SPT, typename KF, typename... A>
void launch_chunks_slots(int64_t n, hipStream_t st, KF k, A... args) {
  const int64_t K = (n + C - 1) / C;
  if (K > 0) hipLaunchKernelGGL(k, dim3((unsigned)K), dim3(Geo<C, SPT>::T), 0, st, n / C, args...);
}

// The same with `lds` bytes of dynamic LDS per workgroup that the kernel
// does not use: it caps the workgroups a CU holds at once (160 KiB each).
template <int C, typename KF, typename... A>
void launch_chunks_capped(unsigned lds, int64_t n, hipStream_t st, KF k, A... args) {
  const int64_t K = (n + C - 1) / C;
  if (K > 0) hipLaunchKernelGGL(k, dim3((unsigned)K), dim3(Geo<C>::T), lds, st, n / C, args...);
}

// Tuning of the compression-step kernels, measured on MI355X at the
// BERT-Large table with W = 8 (phase 1, interleaved medians on one machine:
// plain accesses 7.76 ms, streaming 7.38 ms; with the partial chunk folded
// into the grid, streaming with a 6-wave register cap 7.05 ms, uncapped 7.39,
// 7-wave cap 7.44, 8-wave cap 7.89 -- the cap's spills are reloaded every
// worker iteration, so the best cap depends on where they land; prefetching
// the next worker, keeping beta1*m in LDS, or keeping the workers' signs in
// LDS and summing after the loop (no spills, 3.5% slower) did not help; a
// persistent grid of one workgroup per CU that loads only the next chunk's
// m, g_0 and e_0 across the current chunk's server reduction came within 1%,
// and was slower at other grid sizes or with contiguous chunk ranges).
constexpr bool kPassA_NT = true;   // streaming loads and stores
constexpr bool kPassA_PF = false;  // next-worker prefetch
constexpr int kPassA_WPE = 6;      // minimum waves per SIMD
// A table of at most 16 chunks per CU takes pass A at four waves per SIMD:
// six leave the last of its 2.7 rounds (4096 chunks, 256 CUs) part empty.
// Single 16M-element tensor, W = 4, three interleaved pairs on one machine:
// 0.262 against 0.269 ms per step (packed momentum 0.236 against 0.251);
// on the BERT-XL table (W = 4) four were 2-4% slower in phase 1.
constexpr int kPassA_WPE_small = 4;
constexpr int64_t kPassA_small_per_cu = 16;
// Float4 slots per thread of pass A (workgroup = C / (4 * SPT)): the chunk's
// own layout, four from 1024 elements up.
template <int C>
constexpr int kPassA_SPT = kSlots<C>;
// With 4096-element chunks and at least kPassA_ring_min_W workers, pass A
// runs as a persistent grid with two workers and the next chunk's first
// three in flight (k_compressed_pass_a_ring).  At BERT-Large, W = 8,
// interleaved against one workgroup per chunk on seven machines, it was
// 0.7-4.2% faster (7.05-7.16 against 7.16-7.38 ms; the larger gains where
// the 30-stream pattern runs slowest), outputs identical.  Over W on one
// table (two machines): W = 2-6 slower (by 22% at W = 2, 1-4% at W = 4-6: per
// chunk there is too little worker traffic to hide its reductions behind),
// W = 7 even, W = 8-16 between 4.8% faster and 2% slower, 1.1% faster on
// average.  With 2048-element chunks it was 4% slower, with 1024 no faster,
// and larger chunks would need more than one wave per SIMD at its register
// count; all of those keep the layout above.
template <int C>
constexpr bool kPassA_ring = C == 4096;
constexpr int kPassA_ring_min_W = 7;
constexpr bool kPassB_NT = true;
// Pass B at 4096-element chunks runs at most two workgroups per CU: each
// takes 64 KiB of dynamic LDS it does not use, of the CU's 160 KiB.  Fewer
// chunks in flight serve its five streams better (interleaved at
// BERT-Large: 0.870 against 0.901 ms for finalize + pass B; three per CU
// 0.899 ms, one per CU 0.983 ms; outputs identical).
template <int C>
constexpr unsigned kPassB_lds = C == 4096 ? 65536u : 0u;
// LAMB warmup passes (BERT-Large, W = 8, interleaved on one machine): streaming
// accesses take pass 1 from 3.30 to 2.95 ms and pass 2 from 0.97 to 0.87 ms;
// a 5- or 6-wave register cap on pass 1 is slower (3.07, 3.44 ms) and one on
// the 1-bit Adam warmup changes nothing (3.19-3.22 against 3.20 ms).  Pass 1
// keeps the next gradient and then m and v in flight while it sums: the
// carried warmup step 3.53-3.61 against 3.56-3.66 ms (two series, outputs
// identical); a persistent grid of one or two workgroups per CU, or caps on
// the workgroups per CU, did not help.  At 4096-element chunks both passes
// lay a chunk over 512 threads (two float4 slots each; pass 1 82 VGPRs and
// five waves per SIMD, where four slots took 143 VGPRs and three) and pass 1
// keeps two gradients in flight: pass 1 alone took 2.63-2.67 against
// 2.69-2.79 ms at W = 8 and 1.74 against 1.83 ms at W = 4 (two series on one
// machine; m and v identical, the per-segment sums within 1e-12, their order
// being the layout's), and the carried warmup step 3.48 / 3.59 against
// 3.56 / 3.72 ms at W = 8 and 2.58 against 2.65 ms at W = 4 (outputs
// identical).  One slot per thread with one, three or all gradients in
// flight was as fast at W = 8 and slower at W = 4; two slots with one
// gradient in flight, or four slots with two, no faster.
constexpr bool kWarm_NT = true;
template <int C>
constexpr int kWarm_SPT = C == 4096 ? 2 : kSlots<C>;
template <int C>
constexpr int kWarm_DEPTH = C == 4096 ? 2 : 1;
// Standalone codec kernels (N = 333,563,904, W = 8, interleaved): streaming
// accesses take compress_ef from 0.741 to 0.655 ms (77% of 8 TB/s),
// average_packed from 0.554 to 0.535 ms and decompress from 0.247 to 0.240 ms.
constexpr bool kCodec_NT = true;

// The 1-bit Adam allreduce kernel is pass A's compressed allreduce without
// the rescale statistics and takes the same settings.
constexpr bool kAdam_NT = true;
constexpr bool kAdam_PF = false;
constexpr int kAdam_WPE = 6;
template <int C>
constexpr int kAdam_SPT = kSlots<C>;
// Sparse-stage kernel (BERT-Large, W = 8, 1 of 64 blocks, interleaved):
// streaming accesses 6.36 ms against 6.66 ms plain; a 5- or 6-wave register
// cap changes nothing (6.38 ms), so it runs uncapped (104 VGPRs, no spills).
constexpr bool kSparse_NT = true;
// One GPU's share of a W-GPU step: the worker compression and the receiver
// statistics stream like the codec kernels.  The worker compression at
// 4096-element chunks runs at most two workgroups per CU, like pass B
// (0.84 against 0.88 ms at N = 333.6 M, two runs on one machine; the receiver
// statistics were 21% slower so capped, and keep the full grid).
constexpr bool kShare_NT = true;
template <int C>
constexpr unsigned kWorker_lds = C == 4096 ? 65536u : 0u;
// Chunk geometry of the element-wise 1-bit Adam warmup kernel (any chunk
// gives the same result; this one gives 256-thread workgroups).
constexpr int kAdamWarmupChunk = 4096;
// Its layout and gradients in flight, as the LAMB warmup's first pass (x, m
// and v identical; at N = 333.6 M the step moved by 0-0.6%, 3.26-3.29 ms at
// W = 8, on a 10 M-element buffer it was 2-4% faster).
constexpr int kAdamWarmupSPT = 2;
constexpr int kAdamWarmupDepth = 2;

// The per-tensor finalize kernels reduce a tensor's (chunk, tensor) segments
// with one workgroup.  When the table's largest tensor has more segments
// than kFinalizeWideSegs (the BERT-Large embedding has 7,630 at 4096
// elements; at 64 elements a 16M-element tensor has 262,144), every tensor
// gets 1024 threads with up to kFinalizeWideU loads in flight each, else 256
// threads that take their segments one at a time: 256 threads walked the
// embedding's segments in 30 dependent loads each, 11-16 us of every step.
constexpr int64_t kFinalizeWideSegs = 2048;
constexpr int kFinalizeWideU = 16;

// The host's bound on the chunks of one launch (onebit_host::max_chunks)
// assumes these workgroup widths: one 64-wide wave below 1024 elements,
// else C/16 threads (four float4 slots each) for the entry points that take
// n and chunk, and C / (4 * table_slots(C)) for the widest layout a table
// kernel takes, so no grid reaches 2^32 work-items.
template <int C>
constexpr bool launch_widths_bounded() {
  constexpr int64_t codec = onebit_host::chunk_threads(C, 4);
  constexpr int64_t table = onebit_host::chunk_threads(C, onebit_host::table_slots(C));
  return Geo<C>::T <= codec && Geo<C, kAdam_SPT<C>>::T <= codec && Geo<C>::T <= table &&
         Geo<C, kPassA_SPT<C>>::T <= table && Geo<C, kWarm_SPT<C>>::T <= table;
}
static_assert(launch_widths_bounded<64>() && launch_widths_bounded<128>() &&
                  launch_widths_bounded<256>() && launch_widths_bounded<512>() &&
                  launch_widths_bounded<1024>() && launch_widths_bounded<2048>() &&
                  launch_widths_bounded<4096>() && launch_widths_bounded<8192>() &&
                  launch_widths_bounded<16384>(),
              "a launch geometry is wider than the host's chunk bound assumes");
static_assert(Geo<kAdamWarmupChunk, kAdamWarmupSPT>::T <=
                  onebit_host::chunk_threads(kAdamWarmupChunk, kAdamWarmupSPT),
              "the 1-bit Adam warmup's width");

template <int C>
struct LaunchCompress {
  static void run(int64_t n, const float* in, float* err, uint32_t* bits, float* scales,
                  int32_t* status, hipStream_t st) {
    launch_chunks<C>(n, st, k_compress_ef<C, kCodec_NT>, n, in, err, bits, scales, status);
  }
};

template <int C>
struct LaunchAverage {
  static void run(int64_t n, int W, const PackedIn& pin, float* err_s, uint32_t* bits,
                  float* scales, int32_t* status, hipStream_t st) {
    launch_chunks<C>(n, st, k_average_packed<C, kCodec_NT>, n, W, pin, err_s, bits, scales,
                     status);
  }
};

template <int C>
struct LaunchDecompress {
  static void run(int64_t n, const uint32_t* bits, const float* scales, float* out,
                  hipStream_t st) {
    launch_chunks<C>(n, st, k_decompress<C, kCodec_NT>, n, bits, scales, out);
  }
};

// x_sq: NULL (x read in pass 1, nothing carried), or the per-segment sums
// of x^2 carried between steps: read in place of x when x_in is true,
// rewritten for the updated x by pass 2.
template <int C>
struct LaunchWarmup {
  static void run(const onebit_layer_table* t, int W, const Workers& wk, float* x, float* m,
                  float* v, float* c_sum, float* c_out, double* x_sq, bool x_in, const Coef& cf,
                  const Ws& ws, int32_t* status, hipStream_t st) {
    constexpr int S = kWarm_SPT<C>;
    constexpr int D = kWarm_DEPTH<C>;
    if (x_in)
      launch_chunks_slots<C, S>(t->N, st, k_warmup_pass1<C, kWarm_NT, 1, true, S, D>, t->dev, W,
                                wk, (const float*)x, m, v, ws.seg_x, ws.seg_u, cf);
    else
      launch_chunks_slots<C, S>(t->N, st, k_warmup_pass1<C, kWarm_NT, 1, false, S, D>, t->dev, W,
                                wk, (const float*)x, m, v, ws.seg_x, ws.seg_u, cf);
    if (t->max_tseg > kFinalizeWideSegs)
      hipLaunchKernelGGL((k_warmup_finalize<1024, kFinalizeWideU>), dim3((unsigned)t->L),
                         dim3(1024), 0, st, t->dev, (const double*)(x_in ? x_sq : ws.seg_x),
                         (const double*)ws.seg_u, c_sum, ws.c_layer, c_out, cf, status);
    else
      hipLaunchKernelGGL(k_warmup_finalize<256>, dim3((unsigned)t->L), dim3(256), 0, st, t->dev,
                         (const double*)(x_in ? x_sq : ws.seg_x), (const double*)ws.seg_u, c_sum,
                         ws.c_layer, c_out, cf, status);
    if (x_sq)
      launch_chunks_slots<C, S>(t->N, st, k_warmup_pass2<C, kWarm_NT, true, S>, t->dev,
                                (const float*)m, (const float*)v, x, (const float*)ws.c_layer,
                                x_sq, cf);
    else
      launch_chunks_slots<C, S>(t->N, st, k_warmup_pass2<C, kWarm_NT, false, S>, t->dev,
                                (const float*)m, (const float*)v, x, (const float*)ws.c_layer,
                                x_sq, cf);
  }
};

template <int C>
struct LaunchFreeze {
  static void run(const onebit_layer_table* t, int W, const float* v, float* v_fresh,
                  const Workers& wk, float* err_s, hipStream_t st) {
    launch_chunks<C>(t->N, st, k_freeze_elems<C>, t->N, W, v, v_fresh, wk, err_s);
  }
};

template <int C>
struct LaunchPassA {
  static void run(const onebit_layer_table* t, int W, const Workers& wk, float* err_s,
                  const float* m, const float* v_frozen, float* v_fresh, uint32_t* bits_s,
                  float* scales_s, const Coef& cf, bool rho_norm, const Ws& ws, int32_t* status,
                  hipStream_t st) {
    const bool pm = m == nullptr;
    if (rho_norm && pm)
      go<true, true>(t, W, wk, err_s, m, v_frozen, v_fresh, bits_s, scales_s, cf, ws, status, st);
    else if (rho_norm)
      go<true, false>(t, W, wk, err_s, m, v_frozen, v_fresh, bits_s, scales_s, cf, ws, status, st);
    else if (pm)
      go<false, true>(t, W, wk, err_s, m, v_frozen, v_fresh, bits_s, scales_s, cf, ws, status, st);
    else
      go<false, false>(t, W, wk, err_s, m, v_frozen, v_fresh, bits_s, scales_s, cf, ws, status, st);
  }
  template <bool RN, bool PM>
  static void go(const onebit_layer_table* t, int W, const Workers& wk, float* err_s,
                 const float* m, const float* v_frozen, float* v_fresh, uint32_t* bits_s,
                 float* scales_s, const Coef& cf, const Ws& ws, int32_t* status, hipStream_t st) {
    const int64_t n_full = t->N / C;
    if (kPassA_ring<C> && W >= kPassA_ring_min_W) {
      // one wave per SIMD: 4 / (waves per chunk) workgroups per CU, no more
      // than there are full chunks (at least one, for a lone partial chunk)
      int64_t G = (int64_t)t->cus * (4 / Geo<C>::NW);
      if (G > n_full) G = n_full;
      if (G < 1) G = 1;
      if constexpr (kPassA_ring<C>)
        hipLaunchKernelGGL((k_compressed_pass_a_ring<C, kPassA_NT, RN, PM>), dim3((unsigned)G),
                           dim3(Geo<C>::T), 0, st, n_full, t->dev, W, wk, err_s, m, v_frozen,
                           v_fresh, bits_s, scales_s, ws.seg_max, ws.seg_x, ws.seg_u, cf,
                           status);
    } else if (t->K <= kPassA_small_per_cu * t->cus) {
      hipLaunchKernelGGL(
          (k_compressed_pass_a<C, kPassA_NT, kPassA_PF, kPassA_WPE_small, kPassA_SPT<C>, RN, PM>),
          dim3((unsigned)t->K), dim3(Geo<C, kPassA_SPT<C>>::T), 0, st, n_full, t->dev, W, wk,
          err_s, m, v_frozen, v_fresh, bits_s, scales_s, ws.seg_max, ws.seg_x, ws.seg_u, cf,
          status);
    } else {
      hipLaunchKernelGGL(
          (k_compressed_pass_a<C, kPassA_NT, kPassA_PF, kPassA_WPE, kPassA_SPT<C>, RN, PM>),
          dim3((unsigned)t->K), dim3(Geo<C, kPassA_SPT<C>>::T), 0, st, n_full, t->dev, W, wk,
          err_s, m, v_frozen, v_fresh, bits_s, scales_s, ws.seg_max, ws.seg_x, ws.seg_u, cf,
          status);
    }
  }
};

// The 1-bit Adam step: the compressed allreduce, then the update from the
// server's packed output (the same update kernel as one GPU's share).
template <int C>
struct LaunchAdam {
  static void run(int64_t n, int W, const Workers& wk, float* err_s, float* m, float* x,
                  const float* v_frozen, uint32_t* bits_s, float* scales_s, const Coef& cf,
                  int32_t* status, hipStream_t st) {
    const int64_t K = (n + C - 1) / C;
    if (m)
      hipLaunchKernelGGL((k_adam_allreduce<C, kAdam_NT, kAdam_PF, kAdam_WPE, kAdam_SPT<C>>),
                         dim3((unsigned)K), dim3(Geo<C, kAdam_SPT<C>>::T), 0, st, n / C, n, K, W, wk,
                         err_s, (const float*)m, bits_s, scales_s, cf, status);
    else
      hipLaunchKernelGGL((k_adam_allreduce<C, kAdam_NT, kAdam_PF, kAdam_WPE, kAdam_SPT<C>, true>),
                         dim3((unsigned)K), dim3(Geo<C, kAdam_SPT<C>>::T), 0, st, n / C, n, K, W, wk,
                         err_s, (const float*)m, bits_s, scales_s, cf, status);
    launch_chunks<C>(n, st, k_adam_update<C, kAdam_NT>, n, (const uint32_t*)bits_s,
                     (const float*)scales_s, v_frozen, x, m, cf);
  }
};

template <int C>
struct LaunchSparse {
  static void run(const onebit_layer_table* t, int W, int nsel, const int32_t* sel,
                  const Workers& wk, const WorkerVals& wv, float* x, float* m, const float* v_frozen,
                  float* v_fresh, const float* c_avg, float* vals_s, const Coef& cf, int32_t* status,
                  hipStream_t st) {
    hipLaunchKernelGGL((k_sparse_step<C, kSparse_NT>), dim3((unsigned)t->K), dim3(Geo<C>::T), 0, st,
                       t->N / C, t->dev, W, nsel, sel, wk, wv, x, m, v_frozen, v_fresh, c_avg,
                       vals_s, cf, status);
  }
};

template <int C>
struct LaunchWorker {
  static void run(int64_t n, const float* g, float* e, const float* m, const uint32_t* bits_m,
                  const float* scales_m, uint32_t* bits_w, float* scales_w, const Coef& cf,
                  int32_t* status, hipStream_t st) {
    if (m)
      launch_chunks_capped<C>(kWorker_lds<C>, n, st, k_worker_compress<C, kShare_NT, false>, n, g,
                              e, m, bits_m, scales_m, bits_w, scales_w, cf, status);
    else
      launch_chunks_capped<C>(kWorker_lds<C>, n, st, k_worker_compress<C, kShare_NT, true>, n, g,
                              e, m, bits_m, scales_m, bits_w, scales_w, cf, status);
  }
};

template <int C>
struct LaunchStats {
  static void run(const onebit_layer_table* t, const uint32_t* bits_s, const float* scales_s,
                  const float* m, const uint32_t* bits_m, const float* scales_m,
                  const float* v_frozen, float* v_fresh, const Coef& cf, bool rn, const Ws& ws,
                  hipStream_t st) {
    if (rn && !m)
      go<true, true>(t, bits_s, scales_s, m, bits_m, scales_m, v_frozen, v_fresh, cf, ws, st);
    else if (rn)
      go<true, false>(t, bits_s, scales_s, m, bits_m, scales_m, v_frozen, v_fresh, cf, ws, st);
    else if (!m)
      go<false, true>(t, bits_s, scales_s, m, bits_m, scales_m, v_frozen, v_fresh, cf, ws, st);
    else
      go<false, false>(t, bits_s, scales_s, m, bits_m, scales_m, v_frozen, v_fresh, cf, ws, st);
  }
  template <bool RN, bool PM>
  static void go(const onebit_layer_table* t, const uint32_t* bits_s, const float* scales_s,
                 const float* m, const uint32_t* bits_m, const float* scales_m,
                 const float* v_frozen, float* v_fresh, const Coef& cf, const Ws& ws,
                 hipStream_t st) {
    launch_chunks<C>(t->N, st, k_rescale_stats<C, kShare_NT, RN, PM>, t->dev, bits_s, scales_s, m,
                     bits_m, scales_m, v_frozen, v_fresh, ws.seg_max, ws.seg_x, ws.seg_u, cf);
  }
};

template <int C>
struct LaunchAdamUpdate {
  static void run(int64_t n, const uint32_t* bits_s, const float* scales_s, const float* v_frozen,
                  float* x, float* m, const Coef& cf, hipStream_t st) {
    launch_chunks<C>(n, st, k_adam_update<C, kShare_NT>, n, bits_s, scales_s, v_frozen, x, m, cf);
  }
};

template <int C>
struct LaunchSparseWorker {
  static void run(int64_t n, int nsel, const int32_t* sel, const float* g, float* e,
                  const float* m, float* vals, const Coef& cf, hipStream_t st) {
    launch_chunks<C>(n, st, k_sparse_worker<C, kShare_NT>, n, nsel, sel, g, e, m, vals, cf);
  }
};

template <int C>
struct LaunchSparseUpdate {
  static void run(const onebit_layer_table* t, int nsel, const int32_t* sel, const float* vals_s,
                  float* x, float* m, const float* v_frozen, float* v_fresh, const float* c_avg,
                  const Coef& cf, int32_t* status, hipStream_t st) {
    launch_chunks<C>(t->N, st, k_sparse_update<C, kShare_NT>, t->dev, nsel, sel, vals_s, x, m,
                     v_frozen, v_fresh, c_avg, cf, status);
  }
};

// The per-tensor rho, soft thresholds and c of a compression step.
void rescale_finalize(const onebit_layer_table* t, const float* c_avg, float* f_prev,
                      float* c_out, const Coef& cf, bool rho_norm, const Ws& ws, int32_t* status,
                      hipStream_t st) {
  const bool wide = t->max_tseg > kFinalizeWideSegs;
  if (rho_norm && wide)
    hipLaunchKernelGGL((k_rescale_finalize<1024, true, kFinalizeWideU>), dim3((unsigned)t->L),
                       dim3(1024), 0, st, t->dev, (const float*)ws.seg_max,
                       (const double*)ws.seg_x, (const double*)ws.seg_u, c_avg, f_prev,
                       ws.c_layer, c_out, cf, status);
  else if (rho_norm)
    hipLaunchKernelGGL((k_rescale_finalize<256, true>), dim3((unsigned)t->L), dim3(256), 0, st,
                       t->dev, (const float*)ws.seg_max, (const double*)ws.seg_x,
                       (const double*)ws.seg_u, c_avg, f_prev, ws.c_layer, c_out, cf, status);
  else if (wide)
    hipLaunchKernelGGL((k_rescale_finalize<1024, false, kFinalizeWideU>), dim3((unsigned)t->L),
                       dim3(1024), 0, st, t->dev, (const float*)ws.seg_max,
                       (const double*)ws.seg_x, (const double*)ws.seg_u, c_avg, f_prev,
                       ws.c_layer, c_out, cf, status);
  else
    hipLaunchKernelGGL((k_rescale_finalize<256>), dim3((unsigned)t->L), dim3(256), 0, st,
                       t->dev, (const float*)ws.seg_max, (const double*)ws.seg_x,
                       (const double*)ws.seg_u, c_avg, f_prev, ws.c_layer, c_out, cf, status);
}

template <int C>
struct LaunchPassB {
  static void run(const onebit_layer_table* t, const uint32_t* bits_s, const float* scales_s,
                  float* x, float* m, const float* v_frozen, const float* c_avg, float* f_prev,
                  float* c_out, const Coef& cf, bool rho_norm, const Ws& ws, int32_t* status,
                  hipStream_t st) {
    rescale_finalize(t, c_avg, f_prev, c_out, cf, rho_norm, ws, status, st);
    launch_chunks_capped<C>(kPassB_lds<C>, t->N, st, k_compressed_pass_b<C, kPassB_NT>, t->dev,
                            bits_s, scales_s, v_frozen, x, m, (const float*)ws.c_layer, cf);
  }
};

// ---------------------------------------------------------------------------
// Chunks longer than 16384 elements (onebit_big.hpp): one workgroup of 256
// threads per chunk walks it in 4096-element blocks.  The 1-bit LAMB and
// 1-bit Adam compression steps run there as their per-GPU parts in order:
// every worker's compression, the server's average of the workers' packed
// chunks, then the statistics and the update.  Those parts give the fused
// step's results bit for bit; they need the workers' sign words and scales
// kept, and (1-bit LAMB) an fp32 momentum, since the server's new output
// would overwrite a packed momentum before the statistics read it.
// ---------------------------------------------------------------------------
constexpr int32_t kMaxFusedChunk = 16384;
bool big_chunk(int32_t chunk) { return chunk > kMaxFusedChunk; }
int big_lr(int32_t chunk) {
  int lr = 0;
  while ((kBlk << lr) < chunk) ++lr;
  return lr;
}
static_assert(kBT <= onebit_host::chunk_threads(int64_t(kBlk) << kBigMinLog, 4),
              "the host's chunk bound assumes 256 threads per long chunk");

// The compression kernels' form by chunk length: chunks of 2^15 and 2^16
// held in registers (8 or 16 blocks per thread group), longer ones walked
// twice.  f is called with std::integral_constant<int, RES>.
template <class F>
void by_res(int lr, F&& f) {
  if (lr == 3) f(std::integral_constant<int, 8>{});
  else if (lr == 4) f(std::integral_constant<int, 16>{});
  else f(std::integral_constant<int, 0>{});
}

// The launch over the n elements' chunks (nothing for n = 0); lds bytes of
// dynamic LDS cap the workgroups resident on a CU.
template <typename KF, typename... A>
void big_launch_lds(unsigned lds, int64_t n, int32_t chunk, hipStream_t st, KF k, A... args) {
  const int64_t K = onebit_host::chunks_of(n, chunk);
  if (K > 0) hipLaunchKernelGGL(k, dim3((unsigned)K), dim3(kBT), lds, st, args...);
}
template <typename KF, typename... A>
void big_launch(int64_t n, int32_t chunk, hipStream_t st, KF k, A... args) {
  big_launch_lds(0u, n, chunk, st, k, args...);
}
// The update at two workgroups per CU (63 KiB of dynamic LDS each; three
// would need more than the CU's 160 KiB), as the update at 4096: 1.008
// against 1.040 ms uncapped at chunks of 32768 (BERT-Large table).  The
// statistics kernel was 17% slower so capped and keeps no cap.
constexpr unsigned kBigUpdate_lds = 63u * 1024u;

// A compression step over chunks longer than 16384 elements needs the
// workers' sign words and scales (EUNSUPPORTED otherwise) and, with
// need_m, the fp32 momentum.
int check_big_step(const char* fn, int32_t chunk, int32_t W, uint32_t* const* bits_w,
                   float* const* scales_w, const float* m, bool need_m) {
  if (!big_chunk(chunk)) return ONEBIT_OK;
  for (int w = 0; w < W; ++w)
    if (!bits_w || !scales_w || !bits_w[w] || !scales_w[w])
      return fail(ONEBIT_EUNSUPPORTED,
                  "%s: chunks over %d elements need the workers' sign words and scales "
                  "(bits_w, scales_w)", fn, kMaxFusedChunk);
  if (need_m && !m)
    return fail(ONEBIT_EUNSUPPORTED,
                "%s: chunks over %d elements need the fp32 momentum (m = NULL is packed)", fn,
                kMaxFusedChunk);
  return ONEBIT_OK;
}

// The sparse stage keeps chunks of at most 16384 elements.
int sparse_big(const char* fn, int32_t chunk) {
  return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d: the sparse stage takes chunks of at most %d", fn,
              chunk, kMaxFusedChunk);
}

void big_warmup(const onebit_layer_table* t, int W, const Workers& wk, float* x, float* m,
                float* v, float* c_sum, float* c_out, double* x_sq, bool x_in, const Coef& cf,
                const Ws& ws, int32_t* status, hipStream_t st) {
  const int lr = big_lr(t->chunk);
  if (x_in)
    big_launch(t->N, t->chunk, st, k_big_warmup_pass1<kWarm_NT, true>, t->dev, lr, W, wk,
               (const float*)x, m, v, ws.seg_x, ws.seg_u, cf);
  else
    big_launch(t->N, t->chunk, st, k_big_warmup_pass1<kWarm_NT, false>, t->dev, lr, W, wk,
               (const float*)x, m, v, ws.seg_x, ws.seg_u, cf);
  if (t->max_tseg > kFinalizeWideSegs)
    hipLaunchKernelGGL((k_warmup_finalize<1024, kFinalizeWideU>), dim3((unsigned)t->L), dim3(1024),
                       0, st, t->dev, (const double*)(x_in ? x_sq : ws.seg_x),
                       (const double*)ws.seg_u, c_sum, ws.c_layer, c_out, cf, status);
  else
    hipLaunchKernelGGL(k_warmup_finalize<256>, dim3((unsigned)t->L), dim3(256), 0, st, t->dev,
                       (const double*)(x_in ? x_sq : ws.seg_x), (const double*)ws.seg_u, c_sum,
                       ws.c_layer, c_out, cf, status);
  if (x_sq)
    big_launch(t->N, t->chunk, st, k_big_warmup_pass2<kWarm_NT, true>, t->dev, lr,
               (const float*)m, (const float*)v, x, (const float*)ws.c_layer, x_sq, cf);
  else
    big_launch(t->N, t->chunk, st, k_big_warmup_pass2<kWarm_NT, false>, t->dev, lr,
               (const float*)m, (const float*)v, x, (const float*)ws.c_layer, x_sq, cf);
}

// Every worker's compression, then the server's average of their packed
// chunks: the compressed allreduce of both steps (m NULL: packed momentum,
// read from bits_s / scales_s before the server rewrites them).
void big_allreduce(int64_t n, int32_t chunk, int W, const Workers& wk, float* err_s,
                   const float* m, uint32_t* bits_s, float* scales_s, const Coef& cf,
                   int32_t* status, hipStream_t st) {
  const int lr = big_lr(chunk);
  PackedIn pin{};
  // With the fp32 momentum, one launch for all workers (they share m
  // through L2) unless its grid would pass 2^32 work-items.  A packed
  // momentum is 1/32 of m's bytes: there the one launch saved nothing and
  // made the 1-bit Adam step 3% slower (chunks of 32768, W = 8), so each
  // worker keeps its own launch.
  const int64_t K = onebit_host::chunks_of(n, chunk);
  const int64_t groups = (K + 7) / 8 * 8 * W;
  const bool one_launch = m && K > 0 && groups * kBT <= (int64_t)UINT32_MAX;
  by_res(lr, [&](auto R) {
    constexpr int RES = decltype(R)::value;
    if (one_launch)
      hipLaunchKernelGGL((k_big_workers_compress<kShare_NT, RES>), dim3((unsigned)groups),
                         dim3(kBT), 0, st, n, lr, W, wk, m, cf, status);
    for (int w = 0; w < W; ++w) {
      pin.bits[w] = wk.bits[w];
      pin.scales[w] = wk.scales[w];
      if (one_launch) continue;
      if (m)
        big_launch(n, chunk, st, k_big_worker_compress<kShare_NT, false, RES>, n, lr, wk.g[w],
                   wk.e[w], m, (const uint32_t*)nullptr, (const float*)nullptr, wk.bits[w],
                   wk.scales[w], cf, status);
      else
        big_launch(n, chunk, st, k_big_worker_compress<kShare_NT, true, RES>, n, lr, wk.g[w],
                   wk.e[w], m, (const uint32_t*)bits_s, (const float*)scales_s, wk.bits[w],
                   wk.scales[w], cf, status);
    }
    big_launch(n, chunk, st, k_big_average_packed<kCodec_NT, RES>, n, lr, W, pin, err_s, bits_s,
               scales_s, status);
  });
}

void big_stats(const onebit_layer_table* t, const uint32_t* bits_s, const float* scales_s,
               const float* m, const uint32_t* bits_m, const float* scales_m,
               const float* v_frozen, float* v_fresh, const Coef& cf, bool rn, const Ws& ws,
               hipStream_t st) {
  const int lr = big_lr(t->chunk);
#define BIG_STATS(RN, PM)                                                                        \
  big_launch(t->N, t->chunk, st, k_big_rescale_stats<kShare_NT, RN, PM>, t->dev, lr, bits_s,     \
             scales_s, m, bits_m, scales_m, v_frozen, v_fresh, ws.seg_max, ws.seg_x, ws.seg_u, cf)
  if (rn && !m) BIG_STATS(true, true);
  else if (rn) BIG_STATS(true, false);
  else if (!m) BIG_STATS(false, true);
  else BIG_STATS(false, false);
#undef BIG_STATS
}

// 1-bit LAMB pass A: the allreduce, then the fresh variance and the
// rescale statistics
void big_pass_a(const onebit_layer_table* t, int W, const Workers& wk, float* err_s,
                const float* m, const float* v_frozen, float* v_fresh, uint32_t* bits_s,
                float* scales_s, const Coef& cf, bool rn, const Ws& ws, int32_t* status,
                hipStream_t st) {
  big_allreduce(t->N, t->chunk, W, wk, err_s, m, bits_s, scales_s, cf, status, st);
  big_stats(t, bits_s, scales_s, m, nullptr, nullptr, v_frozen, v_fresh, cf, rn, ws, st);
}

// 1-bit LAMB pass B: the per-tensor coefficients, then the update
void big_pass_b(const onebit_layer_table* t, const uint32_t* bits_s, const float* scales_s,
                float* x, float* m, const float* v_frozen, const float* c_avg, float* f_prev,
                float* c_out, const Coef& cf, bool rn, const Ws& ws, int32_t* status,
                hipStream_t st) {
  rescale_finalize(t, c_avg, f_prev, c_out, cf, rn, ws, status, st);
  big_launch_lds(kBigUpdate_lds, t->N, t->chunk, st, k_big_pass_b<kPassB_NT>, t->dev,
                 big_lr(t->chunk), bits_s, scales_s, v_frozen, x, m, (const float*)ws.c_layer,
                 cf);
}

// The workers' arrays of a compression step; fills wk.
int check_workers(const char* fn, int32_t W, const float* const* grads, float* const* err_w,
                  uint32_t* const* bits_w, float* const* scales_w, Workers& wk) {
  if (!grads || !err_w) return fail(ONEBIT_EINVAL, "%s: grads or err_w is NULL", fn);
  wk = Workers{};
  for (int w = 0; w < W; ++w) {
    if (!grads[w] || !err_w[w]) return fail(ONEBIT_EINVAL, "%s: grads[%d] or err_w[%d] is NULL", fn, w, w);
    if (!aligned16(grads[w]) || !aligned16(err_w[w]))
      return fail(ONEBIT_EALIGN, "%s: grads[%d] or err_w[%d] is not 16-byte aligned", fn, w, w);
    wk.g[w] = grads[w];
    wk.e[w] = err_w[w];
    if (bits_w) {
      if (bits_w[w] && !aligned4(bits_w[w]))
        return fail(ONEBIT_EALIGN, "%s: bits_w[%d] is not 4-byte aligned", fn, w);
      wk.bits[w] = bits_w[w];
    }
    if (scales_w) {
      if (scales_w[w] && !aligned4(scales_w[w]))
        return fail(ONEBIT_EALIGN, "%s: scales_w[%d] is not 4-byte aligned", fn, w);
      wk.scales[w] = scales_w[w];
    }
  }
  return ONEBIT_OK;
}

// Checks shared by the 1-bit LAMB compressed-step entry points; fills wk.
int check_phase1(const char* fn, const onebit_layer_table* table, int32_t W,
                 const float* const* grads, float* const* err_w, float* err_s, const float* m,
                 const float* v_frozen, float* v_fresh, uint32_t* const* bits_w,
                 float* const* scales_w, uint32_t* bits_s, float* scales_s,
                 const onebit_hparams* hp, void* ws, Workers& wk) {
  if (int rc = check_table(table, fn)) return rc;
  if (int rc = check_W(W, fn)) return rc;
  if (int rc = check_hparams(hp, fn)) return rc;
  if (int rc = check_workers(fn, W, grads, err_w, bits_w, scales_w, wk)) return rc;
  const void* req[] = {err_s, v_frozen, v_fresh, bits_s, scales_s, ws};
  const char* names[] = {"err_s", "v_frozen", "v_fresh", "bits_s", "scales_s", "ws"};
  const int align[] = {16, 16, 16, 4, 4, 16};
  for (int i = 0; i < 6; ++i) {
    if (!req[i]) return fail(ONEBIT_EINVAL, "%s: %s is NULL", fn, names[i]);
    if (reinterpret_cast<uintptr_t>(req[i]) % align[i])
      return fail(ONEBIT_EALIGN, "%s: %s is not %d-byte aligned", fn, names[i], align[i]);
  }
  if (m && !aligned16(m)) return fail(ONEBIT_EALIGN, "%s: m is not 16-byte aligned", fn);
  return ONEBIT_OK;
}

int check_phase2(const char* fn, const onebit_layer_table* table, const uint32_t* bits_s,
                 const float* scales_s, float* x, float* m, const float* v_frozen,
                 const float* c_avg, float* f_prev, float* c_out, const onebit_hparams* hp,
                 void* ws) {
  if (int rc = check_table(table, fn)) return rc;
  if (int rc = check_hparams(hp, fn)) return rc;
  const void* req[] = {bits_s, scales_s, x, v_frozen, c_avg, f_prev, ws};
  const char* names[] = {"bits_s", "scales_s", "x", "v_frozen", "c_avg", "f_prev", "ws"};
  const int align[] = {4, 4, 16, 16, 16, 16, 16};
  for (int i = 0; i < 7; ++i) {
    if (!req[i]) return fail(ONEBIT_EINVAL, "%s: %s is NULL", fn, names[i]);
    if (reinterpret_cast<uintptr_t>(req[i]) % align[i])
      return fail(ONEBIT_EALIGN, "%s: %s is not %d-byte aligned", fn, names[i], align[i]);
  }
  if (m && !aligned16(m)) return fail(ONEBIT_EALIGN, "%s: m is not 16-byte aligned", fn);
  if (c_out && !aligned16(c_out)) return fail(ONEBIT_EALIGN, "%s: c_out is not 16-byte aligned", fn);
  return ONEBIT_OK;
}

// Both warmup entry points: x_sq NULL carries nothing.
int warmup_step(const char* fn, const onebit_layer_table* table, int32_t W,
                const float* const* grads, float* x, float* m, float* v, float* c_sum,
                float* c_out, double* x_sq, int32_t x_sq_valid, const onebit_hparams* hp, void* ws,
                int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (int rc = check_table(table, fn)) return rc;
  if (int rc = check_W(W, fn)) return rc;
  if (int rc = check_hparams(hp, fn)) return rc;
  if (x_sq_valid != 0 && x_sq_valid != 1)
    return fail(ONEBIT_EINVAL, "%s: x_sq_valid = %d is not 0 or 1", fn, x_sq_valid);
  if (!grads) return fail(ONEBIT_EINVAL, "%s: grads is NULL", fn);
  Workers wk{};
  for (int w = 0; w < W; ++w) {
    if (!grads[w]) return fail(ONEBIT_EINVAL, "%s: grads[%d] is NULL", fn, w);
    if (!aligned16(grads[w])) return fail(ONEBIT_EALIGN, "%s: grads[%d] is not 16-byte aligned", fn, w);
    wk.g[w] = grads[w];
  }
  const void* req[] = {x, m, v, c_sum, ws};
  const char* names[] = {"x", "m", "v", "c_sum", "ws"};
  for (int i = 0; i < 5; ++i) {
    if (!req[i]) return fail(ONEBIT_EINVAL, "%s: %s is NULL", fn, names[i]);
    if (!aligned16(req[i])) return fail(ONEBIT_EALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  if (c_out && !aligned16(c_out)) return fail(ONEBIT_EALIGN, "%s: c_out is not 16-byte aligned", fn);
  if (x_sq && !aligned16(x_sq)) return fail(ONEBIT_EALIGN, "%s: x_sq is not 16-byte aligned", fn);
  const Bytes b(table->N, table->chunk);
  Spans sp;
  sp.add_workers(grads, W, b.elems, false, "grads");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v, b.elems, true, "v");
  sp.add(c_sum, 4 * (int64_t)table->L, true, "c_sum");
  sp.add(c_out, 4 * (int64_t)table->L, true, "c_out");
  sp.add(x_sq, 8 * table->S, true, "x_sq");
  sp.add(ws, (int64_t)ws_bytes(table), true, "ws");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(fn)) return rc;
  // With weight decay the direction needs x itself, so pass 1 reads it and
  // forms its norm as well (the carried value would be the same bits).
  const bool x_in = x_sq && x_sq_valid == 1 && hp->weight_decay == 0.0f;
  if (big_chunk(table->chunk))
    big_warmup(table, (int)W, wk, x, m, v, c_sum, c_out, x_sq, x_in, make_coef(*hp),
               ws_view(table, ws), status, (hipStream_t)stream);
  else
    by_chunk<LaunchWarmup>(table->chunk, table, (int)W, wk, x, m, v, c_sum, c_out, x_sq, x_in,
                           make_coef(*hp), ws_view(table, ws), status, (hipStream_t)stream);
  return launch_status(fn);
}

// The fused compression step of both entry points (ws: the caller's
// workspace, or this device's static scratch).
int compressed_step(const char* fn, const onebit_layer_table* table, int32_t W,
                    const float* const* grads, float* const* err_w, float* err_s, float* x,
                    float* m, const float* v_frozen, float* v_fresh, const float* c_avg,
                    float* f_prev, float* c_out, uint32_t* const* bits_w, float* const* scales_w,
                    uint32_t* bits_s, float* scales_s, const onebit_hparams* hp, void* ws,
                    int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  Workers wk;
  if (int rc = check_phase1(fn, table, W, grads, err_w, err_s, m, v_frozen, v_fresh, bits_w,
                            scales_w, bits_s, scales_s, hp, ws, wk))
    return rc;
  if (int rc = check_phase2(fn, table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev, c_out, hp,
                            ws))
    return rc;
  if (int rc = check_big_step(fn, table->chunk, W, bits_w, scales_w, m, true)) return rc;
  const Bytes b(table->N, table->chunk);
  const int64_t tl = 4 * (int64_t)table->L;
  Spans sp;
  sp.add_workers(grads, W, b.elems, false, "grads");
  sp.add_workers(err_w, W, b.elems, true, "err_w");
  sp.add_workers(bits_w, W, b.words, true, "bits_w");
  sp.add_workers(scales_w, W, b.scales, true, "scales_w");
  sp.add(err_s, b.elems, true, "err_s");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(v_fresh, b.elems, true, "v_fresh");
  sp.add(c_avg, tl, false, "c_avg");
  sp.add(f_prev, tl, true, "f_prev");
  sp.add(c_out, tl, true, "c_out");
  sp.add(bits_s, b.words, true, "bits_s");
  sp.add(scales_s, b.scales, true, "scales_s");
  sp.add(ws, (int64_t)ws_bytes(table), true, "ws");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(fn)) return rc;
  const Coef cf = make_coef(*hp);
  const bool rn = hp->rho_mode == ONEBIT_RHO_NORM_RATIO;
  const Ws wsv = ws_view(table, ws);
  hipStream_t st = (hipStream_t)stream;
  if (big_chunk(table->chunk)) {
    big_pass_a(table, (int)W, wk, err_s, m, v_frozen, v_fresh, bits_s, scales_s, cf, rn, wsv,
               status, st);
    big_pass_b(table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev, c_out, cf, rn, wsv, status,
               st);
  } else {
    by_chunk<LaunchPassA>(table->chunk, table, (int)W, wk, err_s, m, v_frozen, v_fresh, bits_s,
                          scales_s, cf, rn, wsv, status, st);
    by_chunk<LaunchPassB>(table->chunk, table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev,
                          c_out, cf, rn, wsv, status, st);
  }
  return launch_status(fn);
}

// ---------------------------------------------------------------------------
// Scratch of onebit_lamb_compressed_step_noalloc, for callers that cannot
// allocate device memory: the same workspace (per-segment statistics and
// per-tensor coefficients) in a file-scope device array instead of the
// caller's buffer.  Every GPU the library runs on holds its own copy for the
// life of the process.  In host code `scratch` only names the variable:
// its device address on the current device comes from hipGetSymbolAddress,
// looked up once per device (when a layer table is made there, else at the
// entry point's first call) and kept here, and only that address is ever
// handed to a kernel.  Every word the step reads from it is written earlier
// in the same step, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out, const char* fn) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
    return fail(ONEBIT_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ONEBIT_EUNSUPPORTED, "%s: device %d beyond the %d this entry point serves", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ONEBIT_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ONEBIT_OK;
}

}  // namespace

extern "C" {

const char* onebit_last_error(void) { return onebit_host::last_error_slot().c_str(); }

const char* onebit_version(void) { return "onebit 0.1 (gfx950)"; }

int onebit_layer_table_create(const int64_t* numels, int32_t L, int32_t chunk,
                              onebit_layer_table** out) {
  if (!numels || !out) return fail(ONEBIT_EINVAL, "%s: NULL argument", __func__);
  *out = nullptr;
  int64_t N = 0, K = 0;
  if (int rc = onebit_host::table_sizes(numels, L, chunk, &N, &K, __func__)) return rc;
  int device = -1;
  if (hipError_t e = hipGetDevice(&device); e != hipSuccess)
    return fail(ONEBIT_EHIP, "%s: hipGetDevice: %s", __func__, hipGetErrorString(e));
  int cus = 0;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
      e != hipSuccess || cus < 1)
    return fail(ONEBIT_EHIP, "%s: compute unit count: %s", __func__,
                e != hipSuccess ? hipGetErrorString(e) : "none");
  // Set-up for onebit_lamb_compressed_step_noalloc on this device: its
  // scratch address is looked up here, outside any stream capture, since
  // every call of it takes a table made on its device.  A failure is left
  // for that entry point to report.
  {
    void* p = nullptr;
    (void)scratch_address(&p, __func__);
  }
  onebit_host::HostTable ht;
  if (int rc = onebit_host::build_table(numels, L, chunk, ht, __func__)) return rc;
  const std::vector<int64_t>& off = ht.off;
  const std::vector<int32_t>& l0 = ht.l0;
  const std::vector<int32_t>& l1 = ht.l1;
  const std::vector<int32_t>& seg = ht.seg;
  const std::vector<int32_t>& lseg = ht.lseg;
  const int64_t S = ht.S;

  onebit_layer_table* t = new (std::nothrow) onebit_layer_table();
  if (!t) return fail(ONEBIT_ENOMEM, "%s: host allocation failed", __func__);
  t->L = L;
  t->chunk = chunk;
  t->N = N;
  t->K = K;
  t->S = S;
  t->device = device;
  t->cus = cus;
  for (int32_t l = 0; l < L; ++l)
    t->max_tseg = std::max<int64_t>(t->max_tseg, (int64_t)lseg[l + 1] - lseg[l]);
  using onebit_host::round256;
  const size_t b_off = round256(sizeof(int64_t) * ((size_t)L + 1));
  const size_t b_k = round256(sizeof(int32_t) * (size_t)K);
  const size_t b_l = round256(sizeof(int32_t) * ((size_t)L + 1));
  const size_t total = b_off + 3 * b_k + b_l;
  hipError_t e = hipMalloc(&t->dblock, total);
  if (e != hipSuccess) {
    delete t;
    return fail(e == hipErrorOutOfMemory ? ONEBIT_ENOMEM : ONEBIT_EHIP, "%s: hipMalloc: %s",
                __func__, hipGetErrorString(e));
  }
  char* p = static_cast<char*>(t->dblock);
  struct Piece {
    const void* src;
    size_t bytes;
    size_t at;
  } pieces[] = {{off.data(), sizeof(int64_t) * ((size_t)L + 1), 0},
                {l0.data(), sizeof(int32_t) * (size_t)K, b_off},
                {l1.data(), sizeof(int32_t) * (size_t)K, b_off + b_k},
                {seg.data(), sizeof(int32_t) * (size_t)K, b_off + 2 * b_k},
                {lseg.data(), sizeof(int32_t) * ((size_t)L + 1), b_off + 3 * b_k}};
  for (const Piece& pc : pieces) {
    e = hipMemcpy(p + pc.at, pc.src, pc.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(t->dblock);
      delete t;
      return fail(ONEBIT_EHIP, "%s: hipMemcpy: %s", __func__, hipGetErrorString(e));
    }
  }
  t->dev.off = reinterpret_cast<const int64_t*>(p);
  t->dev.l0 = reinterpret_cast<const int32_t*>(p + b_off);
  t->dev.l1 = reinterpret_cast<const int32_t*>(p + b_off + b_k);
  t->dev.seg = reinterpret_cast<const int32_t*>(p + b_off + 2 * b_k);
  t->dev.lseg = reinterpret_cast<const int32_t*>(p + b_off + 3 * b_k);
  t->dev.N = N;
  t->dev.K = K;
  t->dev.L = L;
  *out = t;
  return ok();
}

int onebit_layer_table_destroy(onebit_layer_table* table) {
  if (!table) return ok();
  hipError_t e = hipSuccess;
  if (table->dblock) e = hipFree(table->dblock);
  delete table;
  if (e != hipSuccess) return fail(ONEBIT_EHIP, "%s: hipFree: %s", __func__, hipGetErrorString(e));
  return ok();
}

int onebit_layer_table_info(const onebit_layer_table* table, int64_t* N, int64_t* K,
                            int64_t* n_segments) {
  if (int rc = check_table(table, __func__)) return rc;
  if (N) *N = table->N;
  if (K) *K = table->K;
  if (n_segments) *n_segments = table->S;
  return ok();
}

int onebit_workspace_size(const onebit_layer_table* table, int32_t W, size_t* bytes) {
  if (int rc = check_table(table, __func__)) return rc;
  if (int rc = check_W(W, __func__)) return rc;
  if (!bytes) return fail(ONEBIT_EINVAL, "%s: bytes is NULL", __func__);
  *bytes = ws_bytes(table);
  return ok();
}

int onebit_compress_ef(int64_t n, int32_t chunk, const float* in, float* err, uint32_t* bits,
                       float* scales, int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (n == 0) return ok();
  CHECK_PTR(in, "in");
  CHECK_PTR(err, "err");
  CHECK_WORDS(bits, "bits");
  CHECK_WORDS(scales, "scales");
  const Bytes b(n, chunk);
  Spans sp;
  sp.add(in, b.elems, false, "in");
  sp.add(err, b.elems, true, "err");
  sp.add(bits, b.words, true, "bits");
  sp.add(scales, b.scales, true, "scales");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(chunk))
    by_res(big_lr(chunk), [&](auto R) {
      big_launch(n, chunk, (hipStream_t)stream, k_big_compress_ef<kCodec_NT, decltype(R)::value>,
                 n, big_lr(chunk), in, err, bits, scales, status);
    });
  else
    by_chunk<LaunchCompress>(chunk, n, in, err, bits, scales, status, (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_average_packed(int64_t n, int32_t chunk, int32_t W, const uint32_t* const* bits_w,
                          const float* const* scales_w, float* err_s, uint32_t* bits_out,
                          float* scales_out, int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (int rc = check_W(W, __func__)) return rc;
  if (n == 0) return ok();
  if (!bits_w || !scales_w) return fail(ONEBIT_EINVAL, "%s: worker arrays are NULL", __func__);
  PackedIn pin{};
  for (int w = 0; w < W; ++w) {
    CHECK_WORDS(bits_w[w], "bits_w[w]");
    CHECK_WORDS(scales_w[w], "scales_w[w]");
    pin.bits[w] = bits_w[w];
    pin.scales[w] = scales_w[w];
  }
  CHECK_PTR(err_s, "err_s");
  CHECK_WORDS(bits_out, "bits_out");
  CHECK_WORDS(scales_out, "scales_out");
  const Bytes b(n, chunk);
  Spans sp;
  sp.add_workers(bits_w, W, b.words, false, "bits_w");
  sp.add_workers(scales_w, W, b.scales, false, "scales_w");
  sp.add(err_s, b.elems, true, "err_s");
  sp.add(bits_out, b.words, true, "bits_out");
  sp.add(scales_out, b.scales, true, "scales_out");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(chunk))
    by_res(big_lr(chunk), [&](auto R) {
      big_launch(n, chunk, (hipStream_t)stream, k_big_average_packed<kCodec_NT, decltype(R)::value>,
                 n, big_lr(chunk), (int)W, pin, err_s, bits_out, scales_out, status);
    });
  else
    by_chunk<LaunchAverage>(chunk, n, (int)W, pin, err_s, bits_out, scales_out, status,
                            (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_decompress(int64_t n, int32_t chunk, const uint32_t* bits, const float* scales,
                      float* out, void* stream) {
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (n == 0) return ok();
  CHECK_WORDS(bits, "bits");
  CHECK_WORDS(scales, "scales");
  CHECK_PTR(out, "out");
  const Bytes b(n, chunk);
  Spans sp;
  sp.add(bits, b.words, false, "bits");
  sp.add(scales, b.scales, false, "scales");
  sp.add(out, b.elems, true, "out");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(chunk))
    big_launch(n, chunk, (hipStream_t)stream, k_big_decompress<kCodec_NT>, n, big_lr(chunk), bits,
               scales, out);
  else
    by_chunk<LaunchDecompress>(chunk, n, bits, scales, out, (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_lamb_warmup_step(const onebit_layer_table* table, int32_t W, const float* const* grads,
                            float* x, float* m, float* v, float* c_sum, float* c_out,
                            const onebit_hparams* hp, void* ws, int32_t* status, void* stream) {
  return warmup_step(__func__, table, W, grads, x, m, v, c_sum, c_out, nullptr, 0, hp, ws, status,
                     stream);
}

int onebit_lamb_warmup_step_carry(const onebit_layer_table* table, int32_t W,
                                  const float* const* grads, float* x, float* m, float* v,
                                  float* c_sum, float* c_out, double* x_sq, int32_t x_sq_valid,
                                  const onebit_hparams* hp, void* ws, int32_t* status,
                                  void* stream) {
  if (!x_sq) return fail(ONEBIT_EINVAL, "%s: x_sq is NULL", __func__);
  return warmup_step(__func__, table, W, grads, x, m, v, c_sum, c_out, x_sq, x_sq_valid, hp, ws,
                     status, stream);
}

int onebit_lamb_freeze(const onebit_layer_table* table, int32_t W, const float* v, float* v_fresh,
                       float* const* err_w, float* err_s, const float* c_sum, int32_t T_w,
                       float* c_avg, float* f_prev, const onebit_hparams* hp, void* stream) {
  if (int rc = check_table(table, __func__)) return rc;
  if (int rc = check_W(W, __func__)) return rc;
  if (T_w < 1) return fail(ONEBIT_EINVAL, "%s: T_w = %d < 1", __func__, T_w);
  if (hp)
    if (int rc = check_hparams(hp, __func__)) return rc;
  // mean of the warmup coefficients, or the bias correction of their EMA
  const double d = hp ? (double)hp->c_avg_decay : 0.0;
  const float den = d > 0.0 ? (float)(1.0 - std::pow(d, (double)T_w)) : (float)T_w;
  if (!err_w) return fail(ONEBIT_EINVAL, "%s: err_w is NULL", __func__);
  Workers wk{};
  for (int w = 0; w < W; ++w) {
    CHECK_PTR(err_w[w], "err_w[w]");
    wk.e[w] = err_w[w];
  }
  CHECK_PTR(v, "v");
  CHECK_PTR(v_fresh, "v_fresh");
  CHECK_PTR(err_s, "err_s");
  CHECK_PTR(c_sum, "c_sum");
  CHECK_PTR(c_avg, "c_avg");
  CHECK_PTR(f_prev, "f_prev");
  const Bytes b(table->N, table->chunk);
  const int64_t tl = 4 * (int64_t)table->L;
  Spans sp;
  sp.add(v, b.elems, false, "v");
  sp.add(v_fresh, b.elems, true, "v_fresh");
  sp.add_workers(err_w, W, b.elems, true, "err_w");
  sp.add(err_s, b.elems, true, "err_s");
  sp.add(c_sum, tl, false, "c_sum");
  sp.add(c_avg, tl, true, "c_avg");
  sp.add(f_prev, tl, true, "f_prev");
  if (int rc = sp.check(__func__)) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (big_chunk(table->chunk))   // element-wise: any chunk layout gives the same result
    launch_chunks<kBlk>(table->N, st, k_freeze_elems<kBlk>, table->N, (int)W, v, v_fresh, wk,
                        err_s);
  else
    by_chunk<LaunchFreeze>(table->chunk, table, (int)W, v, v_fresh, wk, err_s, st);
  hipLaunchKernelGGL(k_freeze_tensors, dim3((unsigned)((table->L + 255) / 256)), dim3(256), 0, st,
                     (int)table->L, c_sum, den, c_avg, f_prev);
  return launch_status(__func__);
}

int onebit_lamb_compress_average(const onebit_layer_table* table, int32_t W,
                                 const float* const* grads, float* const* err_w, float* err_s,
                                 const float* m, const float* v_frozen, float* v_fresh,
                                 uint32_t* const* bits_w, float* const* scales_w, uint32_t* bits_s,
                                 float* scales_s, const onebit_hparams* hp, void* ws,
                                 int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  Workers wk;
  if (int rc = check_phase1(__func__, table, W, grads, err_w, err_s, m, v_frozen, v_fresh, bits_w,
                            scales_w, bits_s, scales_s, hp, ws, wk))
    return rc;
  const Bytes b(table->N, table->chunk);
  Spans sp;
  sp.add_workers(grads, W, b.elems, false, "grads");
  sp.add_workers(err_w, W, b.elems, true, "err_w");
  sp.add_workers(bits_w, W, b.words, true, "bits_w");
  sp.add_workers(scales_w, W, b.scales, true, "scales_w");
  sp.add(err_s, b.elems, true, "err_s");
  sp.add(m, b.elems, false, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(v_fresh, b.elems, true, "v_fresh");
  sp.add(bits_s, b.words, true, "bits_s");
  sp.add(scales_s, b.scales, true, "scales_s");
  sp.add(ws, (int64_t)ws_bytes(table), true, "ws");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  if (int rc = check_big_step(__func__, table->chunk, W, bits_w, scales_w, m, true)) return rc;
  if (big_chunk(table->chunk))
    big_pass_a(table, (int)W, wk, err_s, m, v_frozen, v_fresh, bits_s, scales_s, make_coef(*hp),
               hp->rho_mode == ONEBIT_RHO_NORM_RATIO, ws_view(table, ws), status,
               (hipStream_t)stream);
  else
    by_chunk<LaunchPassA>(table->chunk, table, (int)W, wk, err_s, m, v_frozen, v_fresh, bits_s,
                          scales_s, make_coef(*hp), hp->rho_mode == ONEBIT_RHO_NORM_RATIO,
                          ws_view(table, ws), status, (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_lamb_rescale_update(const onebit_layer_table* table, const uint32_t* bits_s,
                               const float* scales_s, float* x, float* m, const float* v_frozen,
                               const float* c_avg, float* f_prev, float* c_out,
                               const onebit_hparams* hp, void* ws, int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (int rc = check_phase2(__func__, table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev, c_out,
                            hp, ws))
    return rc;
  const Bytes b(table->N, table->chunk);
  const int64_t tl = 4 * (int64_t)table->L;
  Spans sp;
  sp.add(bits_s, b.words, false, "bits_s");
  sp.add(scales_s, b.scales, false, "scales_s");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(c_avg, tl, false, "c_avg");
  sp.add(f_prev, tl, true, "f_prev");
  sp.add(c_out, tl, true, "c_out");
  sp.add(ws, (int64_t)ws_bytes(table), true, "ws");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(table->chunk))
    big_pass_b(table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev, c_out, make_coef(*hp),
               hp->rho_mode == ONEBIT_RHO_NORM_RATIO, ws_view(table, ws), status,
               (hipStream_t)stream);
  else
    by_chunk<LaunchPassB>(table->chunk, table, bits_s, scales_s, x, m, v_frozen, c_avg, f_prev,
                          c_out, make_coef(*hp), hp->rho_mode == ONEBIT_RHO_NORM_RATIO,
                          ws_view(table, ws), status, (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_lamb_compressed_step(const onebit_layer_table* table, int32_t W,
                                const float* const* grads, float* const* err_w, float* err_s,
                                float* x, float* m, const float* v_frozen, float* v_fresh,
                                const float* c_avg, float* f_prev, float* c_out,
                                uint32_t* const* bits_w, float* const* scales_w, uint32_t* bits_s,
                                float* scales_s, const onebit_hparams* hp, void* ws,
                                int32_t* status, void* stream) {
  return compressed_step(__func__, table, W, grads, err_w, err_s, x, m, v_frozen, v_fresh, c_avg,
                         f_prev, c_out, bits_w, scales_w, bits_s, scales_s, hp, ws, status, stream);
}

int onebit_lamb_compressed_step_noalloc(const onebit_layer_table* table, int32_t W,
                                        const float* const* grads, float* const* err_w,
                                        float* err_s, float* x, float* m, const float* v_frozen,
                                        float* v_fresh, const float* c_avg, float* f_prev,
                                        float* c_out, uint32_t* const* bits_w,
                                        float* const* scales_w, uint32_t* bits_s, float* scales_s,
                                        const onebit_hparams* hp, int32_t* status, void* stream) {
  if (int rc = check_table(table, __func__)) return rc;
  const size_t need = ws_bytes(table);
  if (need > kScratchBytes)
    return fail(ONEBIT_EUNSUPPORTED,
                "%s: the table needs %zu bytes of scratch, more than the %zu this entry point "
                "holds per device (use onebit_lamb_compressed_step with a workspace)",
                __func__, need, kScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_address(&ws, __func__)) return rc;
  return compressed_step(__func__, table, W, grads, err_w, err_s, x, m, v_frozen, v_fresh, c_avg,
                         f_prev, c_out, bits_w, scales_w, bits_s, scales_s, hp, ws, status, stream);
}

int onebit_worker_compress(int64_t n, int32_t chunk, const float* grad, float* err_w,
                           const float* m, const uint32_t* bits_m, const float* scales_m,
                           uint32_t* bits_w, float* scales_w, const onebit_hparams* hp,
                           int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (n < 0) return fail(ONEBIT_EINVAL, "%s: n < 0", __func__);
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (int rc = check_hparams(hp, __func__)) return rc;
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (n == 0) return ok();
  CHECK_PTR(grad, "grad");
  CHECK_PTR(err_w, "err_w");
  CHECK_WORDS(bits_w, "bits_w");
  CHECK_WORDS(scales_w, "scales_w");
  if (m) {
    CHECK_PTR(m, "m");
  } else {
    if (!bits_m || !scales_m)
      return fail(ONEBIT_EINVAL, "%s: m is NULL and bits_m/scales_m do not give it", __func__);
    CHECK_WORDS(bits_m, "bits_m");
    CHECK_WORDS(scales_m, "scales_m");
  }
  const Bytes b(n, chunk);
  Spans sp;
  sp.add(grad, b.elems, false, "grad");
  sp.add(err_w, b.elems, true, "err_w");
  sp.add(m, b.elems, false, "m");
  sp.add(bits_m, b.words, false, "bits_m");
  sp.add(scales_m, b.scales, false, "scales_m");
  sp.add(bits_w, b.words, true, "bits_w");
  sp.add(scales_w, b.scales, true, "scales_w");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(chunk))
    by_res(big_lr(chunk), [&](auto R) {
      constexpr int RES = decltype(R)::value;
      if (m)
        big_launch(n, chunk, (hipStream_t)stream, k_big_worker_compress<kShare_NT, false, RES>, n,
                   big_lr(chunk), grad, err_w, m, bits_m, scales_m, bits_w, scales_w,
                   make_coef(*hp), status);
      else
        big_launch(n, chunk, (hipStream_t)stream, k_big_worker_compress<kShare_NT, true, RES>, n,
                   big_lr(chunk), grad, err_w, m, bits_m, scales_m, bits_w, scales_w,
                   make_coef(*hp), status);
    });
  else
    by_chunk<LaunchWorker>(chunk, n, grad, err_w, m, bits_m, scales_m, bits_w, scales_w,
                           make_coef(*hp), status, (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_lamb_rescale_stats(const onebit_layer_table* table, const uint32_t* bits_s,
                              const float* scales_s, const float* m, const uint32_t* bits_m,
                              const float* scales_m, const float* v_frozen, float* v_fresh,
                              const onebit_hparams* hp, void* ws, void* stream) {
  if (int rc = check_table(table, __func__)) return rc;
  if (int rc = check_hparams(hp, __func__)) return rc;
  CHECK_WORDS(bits_s, "bits_s");
  CHECK_WORDS(scales_s, "scales_s");
  CHECK_PTR(v_frozen, "v_frozen");
  CHECK_PTR(v_fresh, "v_fresh");
  CHECK_PTR(ws, "ws");
  if (m) {
    CHECK_PTR(m, "m");
  } else {
    if (!bits_m || !scales_m)
      return fail(ONEBIT_EINVAL, "%s: m is NULL and bits_m/scales_m do not give it", __func__);
    CHECK_WORDS(bits_m, "bits_m");
    CHECK_WORDS(scales_m, "scales_m");
  }
  const Bytes b(table->N, table->chunk);
  Spans sp;
  sp.add(bits_s, b.words, false, "bits_s");
  sp.add(scales_s, b.scales, false, "scales_s");
  sp.add(m, b.elems, false, "m");
  sp.add(bits_m, b.words, false, "bits_m");
  sp.add(scales_m, b.scales, false, "scales_m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(v_fresh, b.elems, true, "v_fresh");
  sp.add(ws, (int64_t)ws_bytes(table), true, "ws");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(table->chunk))
    big_stats(table, bits_s, scales_s, m, bits_m, scales_m, v_frozen, v_fresh, make_coef(*hp),
              hp->rho_mode == ONEBIT_RHO_NORM_RATIO, ws_view(table, ws), (hipStream_t)stream);
  else
    by_chunk<LaunchStats>(table->chunk, table, bits_s, scales_s, m, bits_m, scales_m, v_frozen,
                          v_fresh, make_coef(*hp), hp->rho_mode == ONEBIT_RHO_NORM_RATIO,
                          ws_view(table, ws), (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_adam_update(int64_t n, int32_t chunk, const uint32_t* bits_s, const float* scales_s,
                       float* x, float* m, const float* v_frozen, const onebit_hparams* hp,
                       void* stream) {
  if (n < 0) return fail(ONEBIT_EINVAL, "%s: n < 0", __func__);
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (int rc = check_hparams(hp, __func__, false)) return rc;
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (n == 0) return ok();
  CHECK_WORDS(bits_s, "bits_s");
  CHECK_WORDS(scales_s, "scales_s");
  CHECK_PTR(x, "x");
  CHECK_OPT_PTR(m, "m");
  CHECK_PTR(v_frozen, "v_frozen");
  const Bytes b(n, chunk);
  Spans sp;
  sp.add(bits_s, b.words, false, "bits_s");
  sp.add(scales_s, b.scales, false, "scales_s");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  if (int rc = sp.check(__func__)) return rc;
  if (big_chunk(chunk))
    big_launch(n, chunk, (hipStream_t)stream, k_big_adam_update<kShare_NT>, n, big_lr(chunk),
               bits_s, scales_s, v_frozen, x, m, make_coef(*hp));
  else
    by_chunk<LaunchAdamUpdate>(chunk, n, bits_s, scales_s, v_frozen, x, m, make_coef(*hp),
                               (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_sparse_worker(int64_t n, int32_t chunk, int32_t nsel, const int32_t* sel,
                         const float* grad, float* err_w, const float* m, float* vals_w,
                         const onebit_hparams* hp, void* stream) {
  if (n < 0) return fail(ONEBIT_EINVAL, "%s: n < 0", __func__);
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (big_chunk(chunk)) return sparse_big(__func__, chunk);
  if (int rc = check_hparams(hp, __func__, false)) return rc;
  if (nsel < 1 || nsel > chunk / 64)
    return fail(ONEBIT_EINVAL, "%s: nsel = %d outside [1, chunk/64 = %d]", __func__, nsel,
                chunk / 64);
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (n == 0) return ok();
  CHECK_WORDS(sel, "sel");
  CHECK_PTR(grad, "grad");
  CHECK_PTR(err_w, "err_w");
  CHECK_PTR(m, "m");
  CHECK_PTR(vals_w, "vals_w");
  const Bytes b(n, chunk);
  const int64_t K = (n + chunk - 1) / chunk;
  Spans sp;
  sp.add(sel, 4 * K, false, "sel");
  sp.add(grad, b.elems, false, "grad");
  sp.add(err_w, b.elems, true, "err_w");
  sp.add(m, b.elems, false, "m");
  sp.add(vals_w, 4 * K * nsel * 64, true, "vals_w");
  if (int rc = sp.check(__func__)) return rc;
  by_chunk<LaunchSparseWorker>(chunk, n, (int)nsel, sel, grad, err_w, m, vals_w, make_coef(*hp),
                               (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_sparse_average(int64_t count, int32_t W, const float* const* vals_w, float* vals_s,
                          void* stream) {
  if (count < 0 || count % 4) return fail(ONEBIT_EINVAL, "%s: count %lld is not a multiple of 4 >= 0",
                                          __func__, (long long)count);
  if (int rc = check_W(W, __func__)) return rc;
  if (count == 0) return ok();
  if (!vals_w) return fail(ONEBIT_EINVAL, "%s: vals_w is NULL", __func__);
  WorkerVals wv{};
  for (int w = 0; w < W; ++w) {
    CHECK_PTR(vals_w[w], "vals_w[w]");
    wv.v[w] = const_cast<float*>(vals_w[w]);
  }
  CHECK_PTR(vals_s, "vals_s");
  Spans sp;
  sp.add_workers(vals_w, W, 4 * count, false, "vals_w");
  sp.add(vals_s, 4 * count, true, "vals_s");
  if (int rc = sp.check(__func__)) return rc;
  const int64_t count4 = count / 4;
  const int64_t blocks = (count4 + 255) / 256 < 65536 ? (count4 + 255) / 256 : 65536;
  hipLaunchKernelGGL(k_mean_values<kShare_NT>, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, count4, (int)W, wv, vals_s);
  return launch_status(__func__);
}

int onebit_sparse_update(const onebit_layer_table* table, int32_t nsel, const int32_t* sel,
                         const float* vals_s, float* x, float* m, const float* v_frozen,
                         float* v_fresh, const float* c_avg, const onebit_hparams* hp,
                         int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (int rc = check_table(table, __func__)) return rc;
  if (big_chunk(table->chunk)) return sparse_big(__func__, table->chunk);
  if (int rc = check_hparams(hp, __func__, false)) return rc;
  if (nsel < 1 || nsel > table->chunk / 64)
    return fail(ONEBIT_EINVAL, "%s: nsel = %d outside [1, chunk/64 = %d]", __func__, nsel,
                table->chunk / 64);
  CHECK_WORDS(sel, "sel");
  CHECK_PTR(vals_s, "vals_s");
  CHECK_PTR(x, "x");
  CHECK_PTR(m, "m");
  CHECK_PTR(v_frozen, "v_frozen");
  CHECK_PTR(v_fresh, "v_fresh");
  CHECK_PTR(c_avg, "c_avg");
  const Bytes b(table->N, table->chunk);
  Spans sp;
  sp.add(sel, 4 * table->K, false, "sel");
  sp.add(vals_s, 4 * table->K * nsel * 64, false, "vals_s");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(v_fresh, b.elems, true, "v_fresh");
  sp.add(c_avg, 4 * (int64_t)table->L, false, "c_avg");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  by_chunk<LaunchSparseUpdate>(table->chunk, table, (int)nsel, sel, vals_s, x, m, v_frozen, v_fresh,
                               c_avg, make_coef(*hp), status, (hipStream_t)stream);
  return launch_status(__func__);
}

int onebit_adam_warmup_step(int64_t n, int32_t W, const float* const* grads, float* x, float* m,
                            float* v, const onebit_hparams* hp, void* stream) {
  if (n < 0) return fail(ONEBIT_EINVAL, "%s: n < 0", __func__);
  if (int rc = check_W(W, __func__)) return rc;
  if (int rc = check_hparams(hp, __func__, false)) return rc;
  if (int rc = check_n(n, kAdamWarmupChunk, __func__, kAdamWarmupSPT)) return rc;
  if (n == 0) return ok();
  if (!grads) return fail(ONEBIT_EINVAL, "%s: grads is NULL", __func__);
  Workers wk{};
  for (int w = 0; w < W; ++w) {
    CHECK_PTR(grads[w], "grads[w]");
    wk.g[w] = grads[w];
  }
  CHECK_PTR(x, "x");
  CHECK_PTR(m, "m");
  CHECK_PTR(v, "v");
  Spans sp;
  sp.add_workers(grads, W, 4 * n, false, "grads");
  sp.add(x, 4 * n, true, "x");
  sp.add(m, 4 * n, true, "m");
  sp.add(v, 4 * n, true, "v");
  if (int rc = sp.check(__func__)) return rc;
  constexpr int C = kAdamWarmupChunk;
  launch_chunks_slots<C, kAdamWarmupSPT>(n, (hipStream_t)stream,
                                         k_adam_warmup<C, 1, kAdamWarmupSPT, kAdamWarmupDepth>, n,
                                         (int)W, wk, x, m, v, make_coef(*hp));
  return launch_status(__func__);
}

int onebit_adam_compressed_step(int64_t n, int32_t chunk, int32_t W, const float* const* grads,
                                float* const* err_w, float* err_s, float* x, float* m,
                                const float* v_frozen, uint32_t* const* bits_w,
                                float* const* scales_w, uint32_t* bits_s, float* scales_s,
                                const onebit_hparams* hp, int32_t* status, void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (n < 0) return fail(ONEBIT_EINVAL, "%s: n < 0", __func__);
  if (!chunk_supported(chunk)) return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d", __func__, chunk);
  if (int rc = check_W(W, __func__)) return rc;
  if (int rc = check_hparams(hp, __func__, false)) return rc;
  if (int rc = check_n(n, chunk, __func__)) return rc;
  if (n == 0) return ok();
  Workers wk;
  if (int rc = check_workers(__func__, W, grads, err_w, bits_w, scales_w, wk)) return rc;
  CHECK_PTR(err_s, "err_s");
  CHECK_PTR(x, "x");
  CHECK_OPT_PTR(m, "m");
  CHECK_PTR(v_frozen, "v_frozen");
  CHECK_WORDS(bits_s, "bits_s");
  CHECK_WORDS(scales_s, "scales_s");
  const Bytes b(n, chunk);
  Spans sp;
  sp.add_workers(grads, W, b.elems, false, "grads");
  sp.add_workers(err_w, W, b.elems, true, "err_w");
  sp.add_workers(bits_w, W, b.words, true, "bits_w");
  sp.add_workers(scales_w, W, b.scales, true, "scales_w");
  sp.add(err_s, b.elems, true, "err_s");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(bits_s, b.words, true, "bits_s");
  sp.add(scales_s, b.scales, true, "scales_s");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  if (int rc = check_big_step(__func__, chunk, W, bits_w, scales_w, m, false)) return rc;
  if (big_chunk(chunk)) {
    big_allreduce(n, chunk, (int)W, wk, err_s, m, bits_s, scales_s, make_coef(*hp), status,
                  (hipStream_t)stream);
    big_launch(n, chunk, (hipStream_t)stream, k_big_adam_update<kAdam_NT>, n, big_lr(chunk),
               (const uint32_t*)bits_s, (const float*)scales_s, v_frozen, x, m, make_coef(*hp));
  } else {
    by_chunk<LaunchAdam>(chunk, n, (int)W, wk, err_s, m, x, v_frozen, bits_s, scales_s,
                         make_coef(*hp), status, (hipStream_t)stream);
  }
  return launch_status(__func__);
}

int onebit_sparse_compressed_step(const onebit_layer_table* table, int32_t W, int32_t nsel,
                                  const int32_t* sel, const float* const* grads,
                                  float* const* err_w, float* x, float* m, const float* v_frozen,
                                  float* v_fresh, const float* c_avg, float* const* vals_w,
                                  float* vals_s, const onebit_hparams* hp, int32_t* status,
                                  void* stream) {
  CHECK_OPT_WORDS(status, "status");
  if (int rc = check_table(table, __func__)) return rc;
  if (big_chunk(table->chunk)) return sparse_big(__func__, table->chunk);
  if (int rc = check_W(W, __func__)) return rc;
  if (int rc = check_hparams(hp, __func__, false)) return rc;
  if (nsel < 1 || nsel > table->chunk / 64)
    return fail(ONEBIT_EINVAL, "%s: nsel = %d outside [1, chunk/64 = %d]", __func__, nsel,
                table->chunk / 64);
  CHECK_WORDS(sel, "sel");
  Workers wk;
  if (int rc = check_workers(__func__, W, grads, err_w, nullptr, nullptr, wk)) return rc;
  WorkerVals wv{};
  if (vals_w)
    for (int w = 0; w < W; ++w) {
      CHECK_OPT_PTR(vals_w[w], "vals_w[w]");
      wv.v[w] = vals_w[w];
    }
  CHECK_PTR(x, "x");
  CHECK_PTR(m, "m");
  CHECK_PTR(v_frozen, "v_frozen");
  CHECK_PTR(v_fresh, "v_fresh");
  CHECK_PTR(c_avg, "c_avg");
  CHECK_PTR(vals_s, "vals_s");
  const Bytes b(table->N, table->chunk);
  const int64_t vals = 4 * table->K * nsel * 64;
  Spans sp;
  sp.add(sel, 4 * table->K, false, "sel");
  sp.add_workers(grads, W, b.elems, false, "grads");
  sp.add_workers(err_w, W, b.elems, true, "err_w");
  sp.add_workers(vals_w, W, vals, true, "vals_w");
  sp.add(x, b.elems, true, "x");
  sp.add(m, b.elems, true, "m");
  sp.add(v_frozen, b.elems, false, "v_frozen");
  sp.add(v_fresh, b.elems, true, "v_fresh");
  sp.add(c_avg, 4 * (int64_t)table->L, false, "c_avg");
  sp.add(vals_s, vals, true, "vals_s");
  sp.add(status, 4, true, "status");
  if (int rc = sp.check(__func__)) return rc;
  by_chunk<LaunchSparse>(table->chunk, table, (int)W, (int)nsel, sel, wk, wv, x, m, v_frozen,
                         v_fresh, c_avg, vals_s, make_coef(*hp), status, (hipStream_t)stream);
  return launch_status(__func__);
}

}  // extern "C"
