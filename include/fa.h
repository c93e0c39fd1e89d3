/*
 * fa.h -- C ABI of the exact-attention library for AMD MI355X (gfx950).
 *
 * Exact scaled-dot-product attention O = softmax(scale * Q K^T) V, computed
 * tile by tile with the online-softmax rescaling so that no N x N matrix is
 * ever written to device memory, and its gradient, which recomputes the
 * scores and probabilities tile by tile from the saved per-row logsumexp.
 *
 * Sources (the pages this library follows):
 *   [FA]  "Flash Attention" notes (sgdbs.github.io, AI_Infra / GPUKernel):
 *         section 1 (overall structure: tiling, online softmax, recompute),
 *         section 2 (online softmax; the two-block merge of (m, l) and of the
 *         unnormalised output, parts 3 and 4, and the forward loop, part 4.2),
 *         section 3 (recomputation: the saved statistic L = m + log l, part 3;
 *         rebuilding P = exp(S - L), part 4.1; the blocked backward loop,
 *         part 4.2), and the backward-derivation page (dV, dP, dS, dQ, dK in
 *         parts 3-4; the identity rowsum(dP o P) = rowsum(dO o O), part 5;
 *         the complete blocked backward, part 6).
 *   [ASC] "FlashAttention backward: deleting the O(N^2) intermediates, how
 *         can the gradient still be right?" (coreui.cn): the 1/sqrt(d_k)
 *         factor carried into dQ and dK.
 *
 * Conventions shared by every entry point
 *   dtype    FA_F32, FA_F16 or FA_BF16: element type of Q, K, V, O, dO, dQ,
 *            dK and dV. LSE and every float workspace are fp32.
 *   layout   Q, K, V, O, dO, dQ, dK, dV are dense [B, H, N, d] arrays, d
 *            fastest (row n of slice (b, h) starts at ((b*H + h)*N + n)*d).
 *            LSE and D are dense fp32 [B, H, N].
 *   sizes    B >= 1, H >= 1, N >= 1, d in {64, 128}; B*H*N < 2^31 rows and
 *            N*d < 2^31 (one slice within 4 GiB). A tensor may exceed
 *            4 GiB: offsets into whole tensors are 64-bit.
 *   causal   0: every query sees every key. 1: query i sees keys j <= i
 *            (top-left aligned; queries and keys have the same length N).
 *   scale    finite and > 0; the pages use 1/sqrt(d). S = scale * Q K^T.
 *   pointers device pointers (hipMalloc'd or equivalent), 16-byte aligned,
 *            owned by the caller. Outputs must not overlap inputs. The
 *            library allocates, frees and synchronises nothing.
 *   stream   a hipStream_t passed as void*; NULL means the null stream.
 *            All work is enqueued on it and the call returns at once.
 *   errors   Every entry point returns FA_OK (0) or a negative FA_ERR_*.
 *            Arguments are checked before anything is enqueued; on an
 *            argument error nothing is enqueued. FA_ERR_LAUNCH reports a
 *            failed kernel launch (hipGetLastError after the launch); faults
 *            inside a kernel surface at the caller's next synchronisation.
 *            No C++ exception crosses this interface. Apart from
 *            fa_bwd_noalloc's per-device scratch (see there) and a
 *            thread-safe per-device cache of its address, the library keeps
 *            no state between calls; it may be called from several threads.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7

/* element types */
#define FA_F32 0
#define FA_F16 1
#define FA_BF16 2

/* status codes */
#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1) /* null or misaligned pointer, size <= 0,
                                   scale not finite and > 0, causal not 0/1,
                                   B*H*N or N*d too large */
#define FA_ERR_UNSUPPORTED (-2) /* head size d or dtype not built */
#define FA_ERR_WORKSPACE (-3)   /* workspace smaller than required */
#define FA_ERR_LAUNCH (-4)      /* kernel launch failed */
#define FA_ERR_SCRATCH (-5)     /* fa_bwd_noalloc: B*H*N above
                                   FA_BWD_NOALLOC_MAX_ROWS */

/* Rows (B*H*N) of the static scratch behind fa_bwd_noalloc. */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)

/* Version of this interface (FA_ABI_VERSION). */
int fa_abi_version(void);

/* Static, human-readable name of a status code. */
const char *fa_status_str(int status);

/*
 * Forward: O = softmax(scale * Q K^T) V per (batch, head) slice, and
 * LSE_i = log sum_j exp(scale * q_i . k_j) (natural log, over the keys row i
 * sees) -- [FA] section 2, part 4.2 (one pass over the key/value tiles with
 * the (m, l, O~) rescaling, division by l deferred to the end) and section 3,
 * part 3 (L = m + log l is the only statistic kept for the backward).
 *
 * In:  Q, K, V   [B, H, N, d] dtype
 * Out: O         [B, H, N, d] dtype (rounded to nearest even once, at the end)
 *      LSE       [B, H, N] fp32
 * All dtypes are supported. For FA_F16/FA_BF16 the probabilities are rounded
 * to dtype before the P V product; every sum is accumulated in fp32. For
 * FA_F32 everything stays in fp32. Deterministic: the same inputs give
 * bit-identical O and LSE.
 */
int fa_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
           const void *V, float scale, int causal, void *O, float *LSE,
           void *stream);

/*
 * Split-key forward: the same O and LSE as fa_fwd (up to rounding), with
 * the keys of every row cut into contiguous ranges that separate workgroups
 * sweep, so that slices with few query blocks still fill the chip. Each
 * range gives a partial result (O_s normalised by its own l_s, and LSE_s) in
 * fp32 workspace; fa_lse_merge then folds the parts with the two-block merge
 * of [FA] section 2, parts 3.1 and 4.1 (a part enters as (LSE_s, 1, O_s)).
 *
 * nsplit: 1..64 ranges at most (the key tiles of 64 keys are divided evenly
 *   and no range is empty, so fewer may be used: fa_fwd_splitkv_parts), or 0
 *   to let the library choose from the grid size (which depends on causal:
 *   the unsplit causal forward pairs its query blocks) and the current
 *   device's compute-unit count; keys are split only where the unsplit
 *   forward would leave compute units idle.
 * In/Out: as fa_fwd. dtype FA_F16 or FA_BF16 (FA_F32: FA_ERR_UNSUPPORTED).
 * workspace: at least fa_fwd_splitkv_workspace_bytes(...) bytes, 256-byte
 *   aligned, caller-owned, overwritten: the parts' O [parts, B, H, N, d] and
 *   LSE [parts, B, H, N] in fp32.
 * Enqueues two kernels (the ranges, then the merge), or, when the keys form a
 * single range and N > 1, the kernel of fa_fwd alone (same results as
 * fa_fwd; the workspace must still be of the stated size). Deterministic.
 */
int fa_fwd_splitkv(int dtype, int B, int H, int N, int d, const void *Q,
                   const void *K, const void *V, float scale, int causal,
                   int nsplit, void *O, float *LSE, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Workspace bytes fa_fwd_splitkv needs for these arguments, the same nsplit
 * and causal (0 for arguments it would reject). */
size_t fa_fwd_splitkv_workspace_bytes(int dtype, int B, int H, int N, int d,
                                      int nsplit, int causal);

/* Number of key ranges fa_fwd_splitkv uses for this nsplit and causal (0 if
 * invalid). */
int fa_fwd_splitkv_parts(int B, int H, int N, int nsplit, int causal);

/*
 * Forward of Nq new queries over Nk keys, for streaming use of the online
 * softmax over a cached prefix ([FA] section 2, part 7: the same running
 * (m, l, O~) lets keys arrive in pieces and be cached): token-by-token
 * decoding (Nq = 1) and chunked prefill (Nq > 1). Query i of a slice sits at
 * position Nk - Nq + i, so with causal = 1 it sees keys 0 .. Nk - Nq + i (the
 * cached prefix and the new keys up to itself; requires Nq <= Nk). With
 * causal = 0 every query sees all Nk keys (any Nq).
 * In:  Q [B, H, Nq, d], K and V [B, H, Nk, d] dtype (FA_F16 or FA_BF16).
 * Out: O [B, H, Nq, d] dtype, LSE [B, H, Nq] fp32.
 * Runs as fa_fwd_splitkv does (key ranges swept by separate workgroups, then
 * fa_lse_merge); nsplit and workspace as there, with its own size function.
 * With Nq = 1 (decoding) the ranges run on a vector kernel, P in fp32.
 */
int fa_fwd_kvcache(int dtype, int B, int H, int Nq, int Nk, int d,
                   const void *Q, const void *K, const void *V, float scale,
                   int causal, int nsplit, void *O, float *LSE,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes fa_fwd_kvcache needs for these arguments, the same nsplit
 * and causal (0 for arguments it would reject). */
size_t fa_fwd_kvcache_workspace_bytes(int dtype, int B, int H, int Nq, int Nk,
                                      int d, int nsplit, int causal);

/* Number of key ranges fa_fwd_kvcache uses for this nsplit and causal (0 if
 * invalid). */
int fa_fwd_kvcache_parts(int B, int H, int Nq, int Nk, int nsplit,
                         int causal);

/*
 * Merge of partial attention results over disjoint key sets ([FA] section 2,
 * parts 3.1 and 4.1: the merge of two blocks' (m, l, O~), folded over the
 * parts), for every row r:
 *   LSE_r = log sum_s exp(LSE_sr),   O_r = sum_s exp(LSE_sr - LSE_r) O_sr.
 * In:  O_parts fp32 [parts, rows, d] (each normalised over its own keys),
 *      LSE_parts fp32 [parts, rows]; LSE = -inf marks an empty part.
 * Out: O [rows, d] in dtype (FA_F32, FA_F16 or FA_BF16), LSE fp32 [rows]; a
 *      row whose parts are all empty gets O = 0 and LSE = -inf.
 * parts >= 1, rows >= 1, d in {64, 128}. Pointers as for the other entry
 * points (16-byte aligned, device memory, outputs not overlapping inputs).
 * The parts may come from fa_fwd_splitkv's workspace or from separate calls
 * (for example one per key shard).
 */
int fa_lse_merge(int dtype, int parts, long long rows, int d,
                 const float *O_parts, const float *LSE_parts, void *O,
                 float *LSE, void *stream);

/*
 * Bytes of workspace fa_bwd needs: fp32 D [B, H, N] and fp32 LSE * log2(e)
 * [B, H, N], each rounded up to a multiple of 256. Returns 0 for arguments
 * fa_bwd would reject.
 */
size_t fa_bwd_workspace_bytes(int dtype, int B, int H, int N, int d);

/*
 * Backward: given dO = dLoss/dO, the O and LSE that fa_fwd returned for the
 * same Q, K, V, scale and causal, computes
 *   D  = rowsum(dO o O)                        [FA] derivation page, part 5
 *   P  = exp(scale * Q K^T - LSE)              [FA] section 3, part 4.1
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D)
 *   dQ = scale * dS K,  dK = scale * dS^T Q    [FA] derivation, parts 3-4;
 *                                              [ASC] for the scale
 * tile by tile, never forming an N x N array in device memory.
 *
 * In:  Q, K, V, O, dO  [B, H, N, d] dtype;  LSE [B, H, N] fp32
 * Out: dQ, dK, dV      [B, H, N, d] dtype
 * workspace: device memory of at least fa_bwd_workspace_bytes(...) bytes,
 *   256-byte aligned, owned by the caller; overwritten (no need to clear it).
 * dtype: FA_F16 and FA_BF16 (FA_F32 returns FA_ERR_UNSUPPORTED). P and dS
 * are rounded to dtype before the products that consume them; all sums are
 * fp32. With FA_F16 that rounding bounds |dS| = |P (dP - D)| by the fp16
 * maximum (65504); dP grows with |dO| |V| sqrt(d), so callers with very
 * large upstream gradients scale dO down (as loss scaling does), or beyond
 * the bound the affected gradients become inf or NaN. Deterministic: the same inputs give bit-identical dQ, dK and dV
 * (every output element is summed by one thread in a fixed order).
 * Enqueues fa_bwd_dq_ws (the dQ sweep, which also forms D into the
 * workspace and stores each row's LSE * log2(e) beside it) and then
 * fa_bwd_dkdv_ws (the dK/dV sweep, reading that scaled LSE, the factor its
 * base-2 exponentials would otherwise apply per score); the results equal
 * fa_bwd_preprocess, fa_bwd_dkdv and fa_bwd_dq called in turn, bit for bit.
 */
int fa_bwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
           const void *V, const void *O, const void *dO, const float *LSE,
           float scale, int causal, void *dQ, void *dK, void *dV,
           void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two launches of fa_bwd as two calls, for callers that time or
 * schedule them apart: fa_bwd_dq_ws and then fa_bwd_dkdv_ws, on one
 * workspace and one stream (or with the first complete before the second
 * starts), enqueue exactly what fa_bwd enqueues and give the same dQ, dK
 * and dV, bit for bit.
 *
 * fa_bwd_dq_ws: dQ (the dQ sweep of fa_bwd_dq_d); it also writes D =
 *   rowsum(dO o O) ([FA] derivation page, part 5) and LSE * log2(e) of every
 *   row into the workspace.
 *   In: Q, K, V, O, dO dtype; LSE fp32.  Out: dQ dtype; the workspace.
 * fa_bwd_dkdv_ws: dK, dV (the dK/dV sweep of fa_bwd_dkdv), reading D and
 *   the scaled LSE that fa_bwd_dq_ws wrote into the workspace for the same
 *   Q, K, V, O, dO, LSE, scale and causal.
 *   In: Q, K, V, dO dtype; the workspace.  Out: dK, dV dtype.
 * workspace: at least fa_bwd_workspace_bytes(...) bytes, 256-byte aligned,
 *   owned by the caller; what is in it is internal to the library.
 * Errors as fa_bwd.
 */
int fa_bwd_dq_ws(int dtype, int B, int H, int N, int d, const void *Q,
                 const void *K, const void *V, const void *O, const void *dO,
                 const float *LSE, float scale, int causal, void *dQ,
                 void *workspace, size_t workspace_bytes, void *stream);
int fa_bwd_dkdv_ws(int dtype, int B, int H, int N, int d, const void *Q,
                   const void *K, const void *V, const void *dO, float scale,
                   int causal, void *dK, void *dV, const void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same inputs, outputs, kernels and
 * results as fa_bwd (bit for bit). The fp32 D = rowsum(dO o O) and
 * LSE * log2(e) rows that fa_bwd keeps in the caller's workspace live instead
 * in a static device array of the library, 2 * FA_BWD_NOALLOC_MAX_ROWS floats
 * (32 MiB), one copy per device,
 * allocated when the library's code loads on that device and held until the
 * process ends; its address is looked up on the first call on each device
 * (the device of `stream`; the current device for the null stream).
 * Nothing is allocated or freed, by this call or by the library.
 * Errors: as fa_bwd, plus FA_ERR_SCRATCH when B*H*N exceeds
 *   FA_BWD_NOALLOC_MAX_ROWS (checked before anything is enqueued).
 * Every call on one device shares that device's scratch: calls whose work
 * overlaps on one device (several streams, or threads on one device) race
 * on it and must be serialised by the caller. Nothing in the scratch needs
 * clearing between calls: every row a call reads was written earlier in
 * the same call.
 */
int fa_bwd_noalloc(int dtype, int B, int H, int N, int d, const void *Q,
                   const void *K, const void *V, const void *O, const void *dO,
                   const float *LSE, float scale, int causal, void *dQ,
                   void *dK, void *dV, void *stream);

/*
 * The three stages of fa_bwd, for callers that schedule them separately.
 * fa_bwd_dkdv and fa_bwd_dq only read what fa_bwd_preprocess wrote, so they
 * may run in either order or concurrently (on two streams).
 *
 * fa_bwd_preprocess: Dvec_i = sum_k dO_ik * O_ik in fp32 ([FA] derivation
 *   page, part 5: computed once before the blocked loop, part 6).
 *   In: O, dO [B,H,N,d] dtype.  Out: Dvec [B,H,N] fp32 (caller-owned).
 */
int fa_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O,
                      const void *dO, float *Dvec, void *stream);

/*
 * fa_bwd_dkdv: dK and dV by the blocked backward loop of [FA] (section 3,
 *   part 4.2 and the derivation page, part 6): one workgroup owns a block
 *   of keys, keeps its dK and dV in registers, and walks the query tiles,
 *   recomputing P and dS for each.
 *   In: Q, K, V, dO dtype; LSE, Dvec fp32.  Out: dK, dV dtype.
 */
int fa_bwd_dkdv(int dtype, int B, int H, int N, int d, const void *Q,
                const void *K, const void *V, const void *dO, const float *LSE,
                const float *Dvec, float scale, int causal, void *dK, void *dV,
                void *stream);

/*
 * fa_bwd_dq: dQ = scale * dS K ([FA] derivation page, parts 3-4) with the
 *   loops the other way round: one workgroup owns a block of query rows,
 *   keeps its dQ in registers, and walks the key tiles, recomputing P and
 *   dS for each, so dQ is written once instead of being accumulated across
 *   key blocks.
 *   In: Q, K, V, dO dtype; LSE, Dvec fp32.  Out: dQ dtype.
 */
int fa_bwd_dq(int dtype, int B, int H, int N, int d, const void *Q,
              const void *K, const void *V, const void *dO, const float *LSE,
              const float *Dvec, float scale, int causal, void *dQ,
              void *stream);

/*
 * fa_bwd_dq_d: fa_bwd_dq with D formed in the same sweep instead of read:
 *   each workgroup forms Dvec for its own query rows from O and dO (the
 *   values fa_bwd_preprocess writes, bit for bit: same products, same
 *   summation tree), uses them and stores them, so that fa_bwd_dkdv can
 *   follow it on the same stream without the preprocess pass. (fa_bwd runs
 *   the same sweep as fa_bwd_dq_ws, which also stores each row's scaled LSE
 *   for the dK/dV sweep.)
 *   In: Q, K, V, O, dO dtype; LSE fp32.  Out: dQ dtype; Dvec [B,H,N] fp32.
 */
int fa_bwd_dq_d(int dtype, int B, int H, int N, int d, const void *Q,
                const void *K, const void *V, const void *O, const void *dO,
                const float *LSE, float *Dvec, float scale, int causal,
                void *dQ, void *stream);

/*
 * Standard attention that stores the N x N matrices: the method the pages
 * set tiled attention against ([FA] section 1: S = Q K^T and P = softmax(S)
 * written out whole before O = P V; section 3: the backward that reads the
 * stored P instead of recomputing it). It exists to measure that trade-off
 * on this chip (time and device memory against fa_fwd / fa_bwd); it gives
 * the same results within rounding. Every step is a separate kernel and
 * every N x N intermediate goes through device memory:
 *   forward:  S = scale Q K^T (fp32, -inf where masked), P = softmax(S)
 *             rounded to dtype, O = P V, LSE = log sum_j exp(S_ij);
 *   backward: D = rowsum(dO o O), dV = P^T dO, dS = P o (dO V^T - D)
 *             rounded to dtype, dQ = scale dS K, dK = scale dS^T Q.
 * N x N arrays of a slice are row-major with fa_std_row_stride(N) elements
 * per row (N rounded up to a multiple of 128); the padding columns of P
 * hold zeros. dtype: FA_F16 and FA_BF16 (FA_F32 returns
 * FA_ERR_UNSUPPORTED). Size limit: B*H*N*fa_std_row_stride(N) < 2^38.
 */
int fa_std_row_stride(int N);

/* Bytes of P: dtype [B, H, N, fa_std_row_stride(N)]; 0 if invalid. */
size_t fa_std_p_bytes(int dtype, int B, int H, int N, int d);

/* Forward workspace: S fp32 [B, H, N, row stride]; 0 if invalid. */
size_t fa_std_fwd_workspace_bytes(int dtype, int B, int H, int N, int d);

/* Backward workspace: dS dtype [B, H, N, row stride], then D fp32
 * [B, H, N] (each part rounded up to 256 bytes); 0 if invalid. */
size_t fa_std_bwd_workspace_bytes(int dtype, int B, int H, int N, int d);

/*
 * In:  Q, K, V [B, H, N, d] dtype.
 * Out: O [B, H, N, d] dtype; LSE [B, H, N] fp32; P (at least
 *      fa_std_p_bytes bytes), kept by the caller for fa_std_bwd.
 * workspace: at least fa_std_fwd_workspace_bytes bytes, 256-byte aligned;
 *   overwritten.
 */
int fa_std_fwd(int dtype, int B, int H, int N, int d, const void *Q,
               const void *K, const void *V, float scale, int causal, void *O,
               float *LSE, void *P, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * In:  Q, K, V, O, dO [B, H, N, d] dtype; P as fa_std_fwd wrote it for the
 *      same inputs (it carries the causal mask as zeros).
 * Out: dQ, dK, dV [B, H, N, d] dtype.
 * workspace: at least fa_std_bwd_workspace_bytes bytes, 256-byte aligned;
 *   overwritten.
 */
int fa_std_bwd(int dtype, int B, int H, int N, int d, const void *Q,
               const void *K, const void *V, const void *O, const void *dO,
               const void *P, float scale, void *dQ, void *dK, void *dV,
               void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
