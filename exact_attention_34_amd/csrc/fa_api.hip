// fa_api.hip -- the C ABI declared in include/fa.h: argument checks, workspace
// layout and dispatch to the kernel launchers. Nothing here allocates, frees
// or synchronises; every launch goes to the caller's stream.

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "fa.h"
#include "fa_launch.h"
#include "fa_std_launch.h"

namespace {

constexpr size_t kAlign = 16;
constexpr size_t kWsAlign = 256;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Checks shared by every entry point. Returns FA_OK or an error code.
int check_shape(int dtype, int B, int H, int N, int d, bool bwd) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  // Rows (and so workgroup counts) fit in int; one slice fits in the 32-bit
  // byte range of a buffer resource. Offsets into whole tensors are 64-bit.
  if ((long long)B * H * N >= (1LL << 31) || (long long)N * d >= (1LL << 31))
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (bwd && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_scale_causal(float scale, int causal) {
  if (!(isfinite(scale) && scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

bool tensor_ok(const void *p) { return p != nullptr && aligned(p, kAlign); }
bool vec_ok(const void *p) { return p != nullptr && aligned(p, 4); }

int status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

size_t d_bytes(int B, int H, int N) { return round_up((size_t)B * H * N * sizeof(float), kWsAlign); }

constexpr int kMaxSplit = 64;

// Key ranges for fa_fwd_splitkv / fa_fwd_kvcache when the caller passes 0,
// from the number of workgroups the unsplit launch would run against the
// compute-unit count; ranges keep at least 16 key tiles (shorter ranges do
// not repay the extra kernel and the merge: at B2 H8 N1024 two ranges of 8
// tiles ran 0.017 ms and four of 4 tiles 0.022 ms, against 0.015 ms unsplit).
//  * Nq = Nk (self-attention; one range runs the plain forward): that
//    forward's units, 128-row blocks, paired under the causal mask. Split
//    only below one unit per compute unit: at B1 H4 N8192 d128 non-causal
//    (256 units) two ranges ran 0.132 ms (merge included) against 0.128 ms
//    unsplit; causal (128 pair units) 0.100 against 0.114 ms.
//  * Nq != Nk (new queries over a cache): the split kernel's units (one per
//    slice, range and 128-row block), about two per compute unit (prefill of
//    512 queries over 8192 keys, 32 slices: four ranges, 0.075 ms).
//  * Nq = 1 (decoding, vector kernel, HBM-bound): about one workgroup of
//    four waves per compute unit, ranges of at least 256 keys. Measured at
//    d = 128 over 1 to 64 ranges: K/V read rates peak (5.1-6.0 TB/s) at
//    256-512 workgroups and fall with more (B1 H32 Nk32768: 8 ranges
//    5.10 TB/s, 32 ranges 4.34; B16 H32 Nk8192: 1 range 5.84, 16 ranges 5.66).
int auto_split(int B, int H, int Nq, int Nk, int causal) {
  int cus = 256, dev = 0, v = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
    cus = v;
  const long bh = (long)B * H;
  long ns;
  if (Nq == 1) {
    ns = (cus + bh - 1) / bh;
    if (ns > Nk / 256) ns = Nk / 256;
  } else {
    const long nqb = (Nq + 127) / 128;
    if (Nq == Nk) {
      const long units = bh * (causal ? (nqb + 1) / 2 : nqb);
      ns = (cus + units - 1) / units;
    } else {
      const long units = bh * nqb;
      ns = (2L * cus + units - 1) / units;
    }
    const long tiles = (Nk + 63) / 64;
    if (ns > tiles / 16) ns = tiles / 16;
  }
  if (ns > kMaxSplit) ns = kMaxSplit;
  return ns < 1 ? 1 : (int)ns;
}

// Requested split count -> ranges actually used (0 if invalid).
int resolve_split(int B, int H, int Nq, int Nk, int nsplit, int causal) {
  if (nsplit < 0 || nsplit > kMaxSplit) return 0;
  if (nsplit == 0) nsplit = auto_split(B, H, Nq, Nk, causal);
  return fa::split_parts(Nk, nsplit);
}

// Workspace of the split forward for `parts` ranges and Nq query rows per
// slice: O parts, then LSE parts.
size_t split_o_bytes(int parts, int B, int H, int Nq, int d) {
  return round_up((size_t)parts * B * H * Nq * d * sizeof(float), kWsAlign);
}
size_t split_bytes(int parts, int B, int H, int Nq, int d) {
  return split_o_bytes(parts, B, H, Nq, d) +
         round_up((size_t)parts * B * H * Nq * sizeof(float), kWsAlign);
}

// Shape checks of the cached-prefix forward: Nq new queries over Nk keys.
int check_kv_shape(int dtype, int B, int H, int Nq, int Nk, int d, int causal) {
  int rc = check_shape(dtype, B, H, Nq, d, false);
  if (rc != FA_OK) return rc;
  if ((rc = check_shape(dtype, B, H, Nk, d, false)) != FA_OK) return rc;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (causal == 1 && Nq > Nk) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// The split-key forward of Nq queries over Nk keys (Nq = Nk for the plain
// case), then the merge; arguments already checked except the workspace.
int run_split(int dtype, int B, int H, int Nq, int Nk, int d, const void *Q, const void *K,
              const void *V, float scale, int causal, int nsplit, void *O, float *LSE,
              void *workspace, size_t workspace_bytes, void *stream) {
  if (nsplit < 0 || nsplit > kMaxSplit) return FA_ERR_INVALID_ARG;
  const int req = nsplit == 0 ? auto_split(B, H, Nq, Nk, causal) : nsplit;
  const int parts = fa::split_parts(Nk, req);
  // One workgroup per slice, key range and 128-row query block: at most
  // B*H*Nq/2 + B*H*parts with parts <= min(64, Nk/64), below 2^31 given
  // the row limits that check_shape put on Nq and Nk.
  if (workspace_bytes < split_bytes(parts, B, H, Nq, d)) return FA_ERR_WORKSPACE;
  float *Op = (float *)workspace;
  float *Lp = (float *)((char *)workspace + split_o_bytes(parts, B, H, Nq, d));
  hipStream_t st = (hipStream_t)stream;
  // A single key range: the kernel writes O and LSE itself (the merge of a
  // single part would only copy them).
  const bool direct = parts == 1;
  int rc = status(fa::launch_fwd_split(dtype, B, H, Nq, Nk, d, Q, K, V, scale, causal, req, Op,
                                       Lp, direct ? O : nullptr, direct ? LSE : nullptr, st));
  if (rc != FA_OK || direct) return rc;
  return status(fa::launch_lse_merge(dtype, parts, (long)B * H * Nq, d, Op, Lp, O, LSE, st));
}

// Standard attention: N x N element count per call, or 0 when too large.
size_t std_elems(int B, int H, int N) {
  const size_t e = (size_t)B * H * N * fa::std_row_stride(N);
  return e < (1ULL << 38) ? e : 0;
}
int check_std(int dtype, int B, int H, int N, int d) {
  const int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  return std_elems(B, H, N) ? FA_OK : FA_ERR_INVALID_ARG;
}
size_t std_ds_bytes(int B, int H, int N) { return round_up(std_elems(B, H, N) * 2, kWsAlign); }

// Static scratch of fa_bwd_noalloc: D = rowsum(dO o O) and LSE * log2(e)
// for up to FA_BWD_NOALLOC_MAX_ROWS rows each (32 MiB), one copy per device,
// allocated when the library's code object loads on that device and held
// until the process ends. Host code never uses this name as an address: the
// device address of each device's copy comes from hipGetSymbolAddress
// (scratch_on).
__device__ __attribute__((aligned(256))) float scratch[2 * FA_BWD_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 256;
std::atomic<float *> g_scratch[kMaxDevices];

// The device address of `scratch` on device dev, looked up once per device
// with that device current (the lookup is the same on every call, so two
// threads racing on the first call store the same value).
int scratch_on(int dev, float **out) {
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  float *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
    void *addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (e != hipSuccess || addr == nullptr) return FA_ERR_LAUNCH;
    p = (float *)addr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FA_OK;
}

// The device whose queue `stream` feeds (the current device for the null
// stream): kernels run there, so the scratch must be that device's copy.
int stream_device(hipStream_t st, int *dev) {
  if (st == nullptr) return hipGetDevice(dev) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
  hipDevice_t d = -1;
  if (hipStreamGetDevice(st, &d) != hipSuccess) return FA_ERR_LAUNCH;
  *dev = (int)d;
  return FA_OK;
}

// fa_bwd's two sweeps with D at Dvec and LSE * log2(e) at L2 (already
// checked arguments).
// The two launches of the backward. The dQ sweep forms D itself (as
// fa_bwd_preprocess would) and stores it, with each row's LSE * log2(e), for
// the dK/dV sweep that follows (the same products as the natural-log LSE
// scaled there), which reads both.
int run_bwd_dq(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
               const void *V, const void *O, const void *dO, const float *LSE, float scale,
               int causal, void *dQ, float *Dvec, float *L2, hipStream_t st) {
  return status(fa::launch_bwd_dq_fused(dtype, B, H, N, d, Q, K, V, O, dO, LSE, Dvec, L2, scale,
                                        causal, dQ, st));
}
int run_bwd_dkdv(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                 const void *V, const void *dO, float scale, int causal, void *dK, void *dV,
                 const float *Dvec, const float *L2, hipStream_t st) {
  // LSE itself is not read when L2 is given.
  return status(fa::launch_bwd_dkdv(dtype, B, H, N, d, Q, K, V, dO, nullptr, L2, Dvec, scale,
                                    causal, dK, dV, st));
}
int run_bwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K, const void *V,
            const void *O, const void *dO, const float *LSE, float scale, int causal, void *dQ,
            void *dK, void *dV, float *Dvec, float *L2, hipStream_t st) {
  int rc = run_bwd_dq(dtype, B, H, N, d, Q, K, V, O, dO, LSE, scale, causal, dQ, Dvec, L2, st);
  if (rc != FA_OK) return rc;
  return run_bwd_dkdv(dtype, B, H, N, d, Q, K, V, dO, scale, causal, dK, dV, Dvec, L2, st);
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char *fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head size or dtype";
    case FA_ERR_WORKSPACE: return "workspace too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH: return "problem larger than the static scratch (B*H*N rows)";
    default: return "unknown status";
  }
}

int fa_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K, const void *V,
           float scale, int causal, void *O, float *LSE, void *stream) {
  int rc = check_shape(dtype, B, H, N, d, false);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !vec_ok(LSE))
    return FA_ERR_INVALID_ARG;
  return status(fa::launch_fwd(dtype, B, H, N, d, Q, K, V, scale, causal, O, LSE,
                               (hipStream_t)stream));
}

size_t fa_fwd_splitkv_workspace_bytes(int dtype, int B, int H, int N, int d, int nsplit,
                                      int causal) {
  if (check_shape(dtype, B, H, N, d, false) != FA_OK || dtype == FA_F32) return 0;
  if (causal != 0 && causal != 1) return 0;
  const int parts = resolve_split(B, H, N, N, nsplit, causal);
  if (parts == 0) return 0;
  return split_bytes(parts, B, H, N, d);
}

int fa_fwd_splitkv_parts(int B, int H, int N, int nsplit, int causal) {
  if (B <= 0 || H <= 0 || N <= 0 || (causal != 0 && causal != 1)) return 0;
  return resolve_split(B, H, N, N, nsplit, causal);
}

size_t fa_fwd_kvcache_workspace_bytes(int dtype, int B, int H, int Nq, int Nk, int d,
                                      int nsplit, int causal) {
  if (causal != 0 && causal != 1) return 0;
  if (check_kv_shape(dtype, B, H, Nq, Nk, d, causal) != FA_OK) return 0;
  const int parts = resolve_split(B, H, Nq, Nk, nsplit, causal);
  if (parts == 0) return 0;
  return split_bytes(parts, B, H, Nq, d);
}

int fa_fwd_kvcache_parts(int B, int H, int Nq, int Nk, int nsplit, int causal) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (causal != 0 && causal != 1)) return 0;
  return resolve_split(B, H, Nq, Nk, nsplit, causal);
}

int fa_fwd_kvcache(int dtype, int B, int H, int Nq, int Nk, int d, const void *Q, const void *K,
                   const void *V, float scale, int causal, int nsplit, void *O, float *LSE,
                   void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_kv_shape(dtype, B, H, Nq, Nk, d, causal);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !vec_ok(LSE) ||
      !tensor_ok(workspace))
    return FA_ERR_INVALID_ARG;
  return run_split(dtype, B, H, Nq, Nk, d, Q, K, V, scale, causal, nsplit, O, LSE, workspace,
                   workspace_bytes, stream);
}

int fa_lse_merge(int dtype, int parts, long long rows, int d, const float *O_parts,
                 const float *LSE_parts, void *O, float *LSE, void *stream) {
  if (parts <= 0 || rows <= 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)parts * rows * d >= (1LL << 40) || rows * (d / 4) >= (1LL << 31) * 256LL)
    return FA_ERR_INVALID_ARG;
  if (!tensor_ok(O_parts) || !vec_ok(LSE_parts) || !tensor_ok(O) || !vec_ok(LSE))
    return FA_ERR_INVALID_ARG;
  return status(fa::launch_lse_merge(dtype, parts, (long)rows, d, O_parts, LSE_parts, O, LSE,
                                     (hipStream_t)stream));
}

int fa_fwd_splitkv(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                   const void *V, float scale, int causal, int nsplit, void *O, float *LSE,
                   void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(dtype, B, H, N, d, false);
  if (rc != FA_OK) return rc;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !vec_ok(LSE) ||
      !tensor_ok(workspace))
    return FA_ERR_INVALID_ARG;
  if (N > 1 && resolve_split(B, H, N, N, nsplit, causal) == 1) {
    // One range: the plain forward computes the same rows without the fp32
    // round trip through the workspace and the merge.
    if (workspace_bytes < split_bytes(1, B, H, N, d)) return FA_ERR_WORKSPACE;
    return status(fa::launch_fwd(dtype, B, H, N, d, Q, K, V, scale, causal, O, LSE,
                                 (hipStream_t)stream));
  }
  return run_split(dtype, B, H, N, N, d, Q, K, V, scale, causal, nsplit, O, LSE, workspace,
                   workspace_bytes, stream);
}

size_t fa_bwd_workspace_bytes(int dtype, int B, int H, int N, int d) {
  if (check_shape(dtype, B, H, N, d, true) != FA_OK) return 0;
  return 2 * d_bytes(B, H, N);
}

int fa_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O, const void *dO,
                      float *Dvec, void *stream) {
  const int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  if (!tensor_ok(O) || !tensor_ok(dO) || !vec_ok(Dvec)) return FA_ERR_INVALID_ARG;
  return status(fa::launch_bwd_preprocess(dtype, B, H, N, d, O, dO, Dvec, (hipStream_t)stream));
}

// Checks shared by the two gradient sweeps (everything but the outputs).
static int check_sweep(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                       const void *V, const void *dO, const float *LSE, const float *Dvec,
                       float scale, int causal) {
  int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(dO) || !vec_ok(LSE) ||
      !vec_ok(Dvec))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int fa_bwd_dkdv(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                const void *V, const void *dO, const float *LSE, const float *Dvec, float scale,
                int causal, void *dK, void *dV, void *stream) {
  const int rc = check_sweep(dtype, B, H, N, d, Q, K, V, dO, LSE, Dvec, scale, causal);
  if (rc != FA_OK) return rc;
  if (!tensor_ok(dK) || !tensor_ok(dV)) return FA_ERR_INVALID_ARG;
  return status(fa::launch_bwd_dkdv(dtype, B, H, N, d, Q, K, V, dO, LSE, nullptr, Dvec, scale,
                                    causal, dK, dV, (hipStream_t)stream));
}

int fa_bwd_dq(int dtype, int B, int H, int N, int d, const void *Q, const void *K, const void *V,
              const void *dO, const float *LSE, const float *Dvec, float scale, int causal,
              void *dQ, void *stream) {
  const int rc = check_sweep(dtype, B, H, N, d, Q, K, V, dO, LSE, Dvec, scale, causal);
  if (rc != FA_OK) return rc;
  if (!tensor_ok(dQ)) return FA_ERR_INVALID_ARG;
  return status(fa::launch_bwd_dq(dtype, B, H, N, d, Q, K, V, dO, LSE, Dvec, scale, causal, dQ,
                                  (hipStream_t)stream));
}

int fa_bwd_dq_d(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                const void *V, const void *O, const void *dO, const float *LSE, float *Dvec,
                float scale, int causal, void *dQ, void *stream) {
  const int rc = check_sweep(dtype, B, H, N, d, Q, K, V, dO, LSE, Dvec, scale, causal);
  if (rc != FA_OK) return rc;
  if (!tensor_ok(O) || !tensor_ok(dQ)) return FA_ERR_INVALID_ARG;
  return status(fa::launch_bwd_dq_fused(dtype, B, H, N, d, Q, K, V, O, dO, LSE, Dvec, nullptr,
                                        scale, causal, dQ, (hipStream_t)stream));
}

int fa_bwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K, const void *V,
           const void *O, const void *dO, const float *LSE, float scale, int causal, void *dQ,
           void *dK, void *dV, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !tensor_ok(dO) ||
      !vec_ok(LSE) || !tensor_ok(dQ) || !tensor_ok(dK) || !tensor_ok(dV) ||
      !tensor_ok(workspace))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(dtype, B, H, N, d)) return FA_ERR_WORKSPACE;
  float *Dvec = (float *)workspace;
  float *L2 = (float *)((char *)workspace + d_bytes(B, H, N));
  return run_bwd(dtype, B, H, N, d, Q, K, V, O, dO, LSE, scale, causal, dQ, dK, dV, Dvec, L2,
                 (hipStream_t)stream);
}

int fa_bwd_dq_ws(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                 const void *V, const void *O, const void *dO, const float *LSE, float scale,
                 int causal, void *dQ, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !tensor_ok(dO) ||
      !vec_ok(LSE) || !tensor_ok(dQ) || !tensor_ok(workspace))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(dtype, B, H, N, d)) return FA_ERR_WORKSPACE;
  float *Dvec = (float *)workspace;
  float *L2 = (float *)((char *)workspace + d_bytes(B, H, N));
  return run_bwd_dq(dtype, B, H, N, d, Q, K, V, O, dO, LSE, scale, causal, dQ, Dvec, L2,
                    (hipStream_t)stream);
}

int fa_bwd_dkdv_ws(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                   const void *V, const void *dO, float scale, int causal, void *dK, void *dV,
                   const void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(dO) || !tensor_ok(dK) ||
      !tensor_ok(dV) || !tensor_ok(workspace))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(dtype, B, H, N, d)) return FA_ERR_WORKSPACE;
  const float *Dvec = (const float *)workspace;
  const float *L2 = (const float *)((const char *)workspace + d_bytes(B, H, N));
  return run_bwd_dkdv(dtype, B, H, N, d, Q, K, V, dO, scale, causal, dK, dV, Dvec, L2,
                      (hipStream_t)stream);
}

int fa_bwd_noalloc(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                   const void *V, const void *O, const void *dO, const float *LSE, float scale,
                   int causal, void *dQ, void *dK, void *dV, void *stream) {
  int rc = check_shape(dtype, B, H, N, d, true);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !tensor_ok(dO) ||
      !vec_ok(LSE) || !tensor_ok(dQ) || !tensor_ok(dK) || !tensor_ok(dV))
    return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  hipStream_t st = (hipStream_t)stream;
  int dev = -1;
  float *Dvec = nullptr;
  if ((rc = stream_device(st, &dev)) != FA_OK) return rc;
  if ((rc = scratch_on(dev, &Dvec)) != FA_OK) return rc;
  // Every row of D and of LSE * log2(e) is written by the dQ sweep before
  // the dK/dV sweep reads it, so the scratch needs no clearing.
  return run_bwd(dtype, B, H, N, d, Q, K, V, O, dO, LSE, scale, causal, dQ, dK, dV, Dvec,
                 Dvec + FA_BWD_NOALLOC_MAX_ROWS, st);
}

int fa_std_row_stride(int N) { return N > 0 ? fa::std_row_stride(N) : 0; }

size_t fa_std_p_bytes(int dtype, int B, int H, int N, int d) {
  if (check_std(dtype, B, H, N, d) != FA_OK) return 0;
  return std_elems(B, H, N) * 2;
}

size_t fa_std_fwd_workspace_bytes(int dtype, int B, int H, int N, int d) {
  if (check_std(dtype, B, H, N, d) != FA_OK) return 0;
  return round_up(std_elems(B, H, N) * sizeof(float), kWsAlign);
}

size_t fa_std_bwd_workspace_bytes(int dtype, int B, int H, int N, int d) {
  if (check_std(dtype, B, H, N, d) != FA_OK) return 0;
  return std_ds_bytes(B, H, N) + d_bytes(B, H, N);
}

int fa_std_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K, const void *V,
               float scale, int causal, void *O, float *LSE, void *P, void *workspace,
               size_t workspace_bytes, void *stream) {
  int rc = check_std(dtype, B, H, N, d);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, causal)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !vec_ok(LSE) ||
      !tensor_ok(P) || workspace == nullptr || !aligned(workspace, kWsAlign))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_std_fwd_workspace_bytes(dtype, B, H, N, d)) return FA_ERR_WORKSPACE;
  return status(fa::launch_std_fwd(dtype, B, H, N, d, Q, K, V, scale, causal, (float *)workspace,
                                   P, O, LSE, (hipStream_t)stream));
}

int fa_std_bwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K, const void *V,
               const void *O, const void *dO, const void *P, float scale, void *dQ, void *dK,
               void *dV, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_std(dtype, B, H, N, d);
  if (rc != FA_OK) return rc;
  if ((rc = check_scale_causal(scale, 0)) != FA_OK) return rc;
  if (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O) || !tensor_ok(dO) ||
      !tensor_ok(P) || !tensor_ok(dQ) || !tensor_ok(dK) || !tensor_ok(dV) ||
      workspace == nullptr || !aligned(workspace, kWsAlign))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_std_bwd_workspace_bytes(dtype, B, H, N, d)) return FA_ERR_WORKSPACE;
  float *Dv = (float *)((char *)workspace + std_ds_bytes(B, H, N));
  return status(fa::launch_std_bwd(dtype, B, H, N, d, Q, K, V, O, dO, P, scale, workspace, Dv,
                                   dQ, dK, dV, (hipStream_t)stream));
}

}  // extern "C"
