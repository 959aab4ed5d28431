/*
 * fa.h -- C ABI of libfa.so: FlashAttention-2 style attention forward and backward on one
 * MI355X (gfx950) GPU.
 *
 * Operation (defined in "Systems and Parallelism", CS336 field map, A2, section 1.2-1.3,
 * problems flash_forward and flash_backward): for every (b, h),
 *
 *     S = Q K^T * scale,  causal: key j visible to query i iff j <= i (top-left),
 *     P = row softmax of S over the visible keys,   O = P V,
 *     L_i = logsumexp_j S_ij  (natural log; the only state the backward needs),
 *
 * and the analytic backward with upstream gradient dO,
 *
 *     dV = P^T dO,   dP = dO V^T,   D_i = sum_k dO_ik O_ik,   dS = P o (dP - D),
 *     dQ = scale * dS K,   dK = scale * dS^T Q,
 *
 * where the backward rebuilds P = exp(S - L) from Q, K and L instead of storing it.
 *
 * Layout: every tensor is dense, row-major [B, H, N, d] (element (b,h,n,k) at
 * ((b*H + h)*N + n)*d + k); L is dense [B, H, Nq] float32. Q, dO, O, dQ have N = Nq;
 * K, V, dK, dV have N = Nk. Element type of Q, K, V, O, dO, dQ, dK, dV is `dtype`;
 * accumulation is float32 in every case. Data pointers must be 16-byte aligned.
 *
 * Ownership: every pointer is a device pointer owned by the caller. The library allocates
 * and frees nothing, keeps no state between calls and is re-entrant; the one exception is
 * fa_backward_noalloc, whose workspace is a static device array (see there). Outputs must
 * not alias inputs.
 *
 * Asynchrony: each call validates its arguments on the host, enqueues its kernels on
 * `stream` (NULL means the default stream) and returns. Results are ready
 * once the stream has been synchronised. A fault inside a kernel surfaces at that
 * synchronisation, as for any HIP kernel.
 *
 * Errors: argument problems are reported synchronously, before anything is enqueued:
 *   FA_ERROR_INVALID_VALUE  negative size, Nk == 0 while B*H*Nq > 0, a NULL or misaligned
 *                           pointer that the call would touch, non-finite scale, a bf16
 *                           backward workspace below B * H * Nq * 8 bytes,
 *                           or a forward workspace that is NULL or not 16-byte aligned
 *                           while workspace_bytes > 0;
 *   FA_ERROR_NOT_SUPPORTED  unknown dtype, d not in {16, 32, 64, 128}, or a size above the
 *                           limits below;
 *   FA_ERROR_LAUNCH_FAILED  the HIP runtime rejected a kernel launch.
 * No C++ exception crosses this interface.
 *
 * Limits: Nq, Nk <= 2^22, B*H <= 2^31 - 1 and B*H*(ceil(Nq/32) + ceil(Nk/32)) < 2^24
 * (launch grids count work-items in 32 bits). Any positive Nq, Nk is accepted (ragged
 * tiles are masked); Nq != Nk is allowed. B*H*Nq == 0 makes fa_forward a no-op; in
 * fa_backward, Nq == 0 with Nk > 0 writes dK = dV = 0.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle (the same typedef as <hip/hip_runtime_api.h>, so either
 * header may come first). NULL is the default stream. */
typedef struct ihipStream_t* hipStream_t;

#if defined(__GNUC__) || defined(__clang__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

typedef enum fa_status {
  FA_SUCCESS = 0,
  FA_ERROR_INVALID_VALUE = 1,
  FA_ERROR_NOT_SUPPORTED = 2,
  FA_ERROR_LAUNCH_FAILED = 3,
  FA_ERROR_SCRATCH_TOO_SMALL = 4  /* fa_backward_noalloc: the sizes need more than its array */
} fa_status;

typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,  /* IEEE binary32 in and out                           */
  FA_DTYPE_BF16 = 1  /* bfloat16 in and out; outputs rounded to nearest even */
} fa_dtype;

/*
 * fa_forward -- O = softmax(Q K^T * scale [+ causal mask]) V and L = row logsumexp.
 *
 * Follows problem flash_forward: the kernel walks key tiles with an online softmax
 * (running row max m and row sum l, rescaling the accumulator when m grows), divides by l
 * once at the end and writes L = scale*m + log(l); with is_causal it skips key tiles above
 * the diagonal and masks only the diagonal tiles.
 *
 *   dtype        FA_DTYPE_F32 or FA_DTYPE_BF16
 *   B, H         batch and head counts (>= 0)
 *   Nq, Nk       query and key counts (>= 0)
 *   d            head dimension: 16, 32, 64 or 128
 *   Q            [B,H,Nq,d] dtype, read
 *   K, V         [B,H,Nk,d] dtype, read
 *   is_causal    0: all keys visible; nonzero: key j visible to query i iff j <= i
 *   scale        multiplies Q K^T (finite; usually 1/sqrt(d))
 *   O            [B,H,Nq,d] dtype, written
 *   L            [B,H,Nq] float32, written (natural-log logsumexp of the scaled scores)
 *   stream       hipStream_t or NULL
 *
 * Needs no workspace. Small causal grids, which could use one to spread their work over
 * more of the GPU, run one workgroup per pair of query tiles here; fa_forward_with_workspace
 * is the same call with that workspace.
 */
FA_API fa_status fa_forward(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                            int64_t d, const void* Q, const void* K, const void* V,
                            int is_causal, float scale, void* O, float* L, hipStream_t stream);

/*
 * fa_forward_workspace_bytes -- bytes of device workspace fa_forward_with_workspace can use
 * for these arguments (0 when it needs none, and for arguments it would reject).
 *
 * Small causal bf16 grids (Nq = Nk a multiple of 128, any d, few tiles per head)
 * spread each pair of query tiles over several workgroups so that every CU has work; their
 * partial softmax states go to the workspace and a second launch merges them (the same
 * rescale the online softmax applies between key tiles, problem flash_forward). The size is
 * (Nq/128) * B * H * ways * 2 * (16*ceil(d/32) + 2) * 128 * 4 bytes, with ways in {2, 4, 8}.
 * fp32 grids of few query tiles spread each tile's keys likewise.
 */
FA_API size_t fa_forward_workspace_bytes(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                         int64_t Nk, int64_t d, int is_causal);

/*
 * fa_forward_with_workspace -- fa_forward with a caller-owned device workspace.
 *
 *   workspace    device scratch, 16-byte aligned; may be NULL with workspace_bytes = 0.
 *                With fa_forward_workspace_bytes() bytes, small grids spread their work
 *                over more workgroups; with fewer the call still succeeds and runs as
 *                fa_forward does (same results up to the order of the final merge). The
 *                call overwrites it; concurrent calls must not share one.
 * Every other argument, and the errors, as for fa_forward; in addition a workspace that is
 * NULL or not 16-byte aligned while workspace_bytes > 0 is FA_ERROR_INVALID_VALUE.
 */
FA_API fa_status fa_forward_with_workspace(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                           int64_t Nk, int64_t d, const void* Q, const void* K,
                                           const void* V, int is_causal, float scale, void* O,
                                           float* L, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/*
 * fa_backward_workspace_bytes -- bytes of device workspace fa_backward can use for these
 * sizes (for fp32, and for sizes fa_backward would reject, 0). For bf16 it is
 *   - two floats per query row (B * H * Nq * 8 bytes, the minimum fa_backward accepts): the
 *     preprocessing step's per-row terms L log2(e) and -D, at the start of the workspace;
 *   - plus, for small square grids (Nq = Nk a multiple of 128, at most 1024 64-row tiles),
 *     room for fp32 partial sums: the call then spreads each workgroup's steps over several
 *     workgroups and a second launch adds the partial dQ, dK and dV up
 *     ((Nq/64) * B * H * ways * 3 * 64 * d * 4 bytes, ways in {2, 4, 8}; the larger of the
 *     causal and the non-causal call's ways). With only the minimum, those calls run one
 *     workgroup per tile (slower; results differ only in the order of the final additions).
 * The caller owns the workspace; its contents need no initialisation and are meaningless
 * after the call.
 */
FA_API size_t fa_backward_workspace_bytes(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                   int64_t Nk, int64_t d);

/*
 * fa_backward -- dQ, dK, dV of O = softmax(Q K^T * scale [+ causal mask]) V.
 *
 * Follows problem flash_backward and the two-pass split of section 1.3.3: a preprocessing
 * kernel forms D_i = sum_k dO_ik O_ik (and L_i log2(e)) per query row in the workspace; the
 * main kernel rebuilds P as exp(S - L) from Q, K and the forward's L; one set of its
 * workgroups walks query tiles for each key tile and accumulates dK and dV, another walks
 * key tiles for each query tile and accumulates dQ, so no output is ever updated atomically
 * and the result is bitwise deterministic. The scale appears once in dQ and once in dK.
 *
 *   Q, K, V, is_causal, scale   exactly as given to fa_forward
 *   O, L                        fa_forward's outputs for those inputs
 *   dO                          [B,H,Nq,d] dtype, upstream gradient
 *   dQ                          [B,H,Nq,d] dtype, written
 *   dK, dV                      [B,H,Nk,d] dtype, written
 *   workspace, workspace_bytes  device scratch, 4-byte aligned: at least B * H * Nq * 8
 *                               bytes for bf16 (may be NULL for fp32), and
 *                               fa_backward_workspace_bytes() bytes for the fastest path; it
 *                               must not overlap any other argument, and calls that share
 *                               one workspace must not run concurrently
 *   stream                      hipStream_t or NULL
 */
FA_API fa_status fa_backward(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      const void* Q, const void* K, const void* V, const void* O,
                      const float* L, const void* dO, int is_causal, float scale,
                      void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * fa_backward_preprocess -- the backward's preprocessing step on its own: for every query
 * row, L_i log2(e) and -D_i with D_i = sum_k dO_ik O_ik (problem flash_backward), written
 * to `workspace` for fa_backward_main. fa_backward is this call followed by
 * fa_backward_main on the same stream; callers that want to place or time the two steps
 * separately can make the two calls themselves. Arguments mean what they mean for
 * fa_backward. For fp32, and when B*H*Nq == 0, there is nothing to precompute and the call
 * returns FA_SUCCESS without enqueuing anything.
 */
FA_API fa_status fa_backward_preprocess(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                 int64_t d, const void* O, const float* L, const void* dO,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_backward_main -- everything fa_backward does after fa_backward_preprocess: dQ, dK and
 * dV from Q, K, V, dO and the per-row terms that fa_backward_preprocess left in
 * `workspace` (which must be that call's workspace, unmodified, on the same stream or
 * otherwise ordered after it). Arguments and errors as for fa_backward; O and L are
 * validated as there and read only by the fp32 path.
 */
FA_API fa_status fa_backward_main(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                           int64_t d, const void* Q, const void* K, const void* V,
                           const void* O, const float* L, const void* dO, int is_causal,
                           float scale, void* dQ, void* dK, void* dV, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * fa_backward_atomic_workspace_bytes -- bytes of device workspace fa_backward_atomic needs
 * (0 for fp32 and for sizes it would reject): the two per-row floats of fa_backward, then an
 * fp32 dQ accumulator, B * H * Nq * (2 + d) * 4 bytes in all.
 */
FA_API size_t fa_backward_atomic_workspace_bytes(fa_dtype dtype, int64_t B, int64_t H,
                                                 int64_t Nq, int64_t Nk, int64_t d);

/*
 * fa_backward_atomic -- fa_backward with the other dQ strategy of section 1.3.3: dQ is
 * accumulated with fp32 atomic additions instead of a second pass over the key tiles.
 * After the same preprocessing step, only the dK/dV workgroups run (128 keys each); for
 * every visible 32-row query tile each wave forms its keys' share dS K on the matrix cores
 * and adds it into an fp32 accumulator in the workspace, which a last launch scales and
 * rounds into dQ. Since the order of the atomic additions varies, dQ may differ from run to
 * run in its last bits (dK and dV do not); fa_backward is the deterministic choice.
 *
 * bf16 only: fp32 returns FA_ERROR_NOT_SUPPORTED. Arguments as for fa_backward, except
 * that workspace_bytes must be at least fa_backward_atomic_workspace_bytes() (else
 * FA_ERROR_INVALID_VALUE). Four launches on `stream`: preprocessing, zeroing of the
 * accumulator, main, conversion.
 */
FA_API fa_status fa_backward_atomic(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                    int64_t Nk, int64_t d, const void* Q, const void* K,
                                    const void* V, const void* O, const float* L,
                                    const void* dO, int is_causal, float scale, void* dQ,
                                    void* dK, void* dV, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of the static device array fa_backward_noalloc keeps its workspace in, per GPU. */
#define FA_BACKWARD_NOALLOC_MAX_BYTES ((size_t)32 << 20)

/*
 * fa_backward_noalloc -- fa_backward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments as fa_backward without the workspace, same computation and bitwise the
 * same results as fa_backward given FA_BACKWARD_NOALLOC_MAX_BYTES bytes of workspace. The
 * workspace is instead a file-scope static device array of that size inside the library,
 * one per GPU, which the GPU holds from the first call on it until the process ends; the
 * call itself allocates nothing (no hipMalloc, hipFree or allocating library routine). On
 * the first call on a device the library takes the array's address on that device (the
 * stream's device) with hipGetSymbolAddress and keeps it.
 *
 * Limits: bf16 needs B * H * Nq * 8 bytes of it (the per-row terms); sizes needing more
 * than FA_BACKWARD_NOALLOC_MAX_BYTES return FA_ERROR_SCRATCH_TOO_SMALL before anything is
 * enqueued. Small square grids use the rest for the partial sums that spread their work
 * over more workgroups when those fit, and otherwise run unsplit, as fa_backward does with
 * too little workspace. fp32 uses the array only for those partial sums.
 *
 * Sharing: every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents; a call reads only what it wrote earlier in the same call, so nothing needs
 * clearing. Calls that overlap on one GPU (on different streams, or from several host
 * threads without ordering between their streams) race on the array and must not be
 * issued; calls on one stream are ordered and safe. Errors as for fa_backward, plus
 * FA_ERROR_SCRATCH_TOO_SMALL, and FA_ERROR_LAUNCH_FAILED when the array's address cannot
 * be obtained.
 */
FA_API fa_status fa_backward_noalloc(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                     int64_t Nk, int64_t d, const void* Q, const void* K,
                                     const void* V, const void* O, const float* L,
                                     const void* dO, int is_causal, float scale, void* dQ,
                                     void* dK, void* dV, hipStream_t stream);

/*
 * fa_forward_kernel_name, fa_backward_kernel_name -- the name, as a profiler lists it, of the
 * attention kernel that fa_forward_with_workspace (fa_forward: workspace_bytes = 0) or
 * fa_backward / fa_backward_main with `workspace_bytes` of workspace launch for these
 * arguments, for example "fwd_causal_wide_kernel<64>" (the library's choice of kernel
 * depends on the grid's size and shape, and on the workspace). The launchers take the same
 * decision from the same code. Static storage, never NULL; "" for arguments the calls would
 * reject.
 */
FA_API const char* fa_forward_kernel_name(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                          int64_t Nk, int64_t d, int is_causal,
                                          size_t workspace_bytes);
FA_API const char* fa_backward_kernel_name(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq,
                                           int64_t Nk, int64_t d, int is_causal,
                                           size_t workspace_bytes);

/* fa_status_string -- static, NUL-terminated name of a status code (never NULL). */
FA_API const char* fa_status_string(fa_status status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
