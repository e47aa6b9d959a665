/*
 * fibatt.h -- C ABI of the Fibottention sparse-attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  Fibottention restricts multi-head self-attention to a
 * per-head support set.  Head i (1-based) uses the generalized Fibonacci
 * sequence Fib(a_i, b_i) (f_1 = a, f_2 = b, f_{n+1} = f_n + f_{n-1}) and a
 * window w_i; query j attends key k iff |j - k| is a term of that sequence
 * and |j - k| <= w_i.  Scores are Q_j . K_k / sqrt(d_h) on the support and
 * -inf elsewhere; a softmax over each query row weights the value rows.
 * (Fibottention paper, arXiv 2406.19391, method section: eq. (1) with the
 * -inf indicator, the definition of Omega_w^{Fib(a,b)}, the Wythoff array
 * paragraph for (a_i, b_i) and eq. (3) for the per-head support; the project
 * README's Algorithms 1 and 3 for the sequence loop and the softmax/P.V
 * steps; the 1/sqrt(d_h) scale is that of scaled dot-product attention as
 * restated in the "Dilated Neighborhood Attention Transformer" background.)
 *
 * Conventions shared by every entry point
 *  - Return value: FIBATT_OK (0) or one of the fibatt_status codes.  No entry
 *    point throws or aborts.  On error a message is available from
 *    fibatt_last_error() (per calling thread) and no output is written and no
 *    GPU work is enqueued.
 *  - Tensor layout: Q, K, V, O, dO, dQ, dK, dV are dense row-major
 *    [B, H, N, d_h] (head-major slabs of N rows of d_h elements), except in
 *    fibatt_fwd_strided / fibatt_bwd_strided, which take per-tensor row
 *    strides; LSE and the backward workspace are [B, H, N].  Every tensor
 *    pointer must be 16-byte aligned and outputs must not alias inputs or
 *    each other.
 *  - Ownership: the caller allocates and frees every buffer (device memory
 *    for tensors, host memory for the per-head parameter arrays).  The library
 *    allocates no device memory and keeps no state between calls, except for
 *    the fixed scratch array of fibatt_bwd_noalloc (one per GPU, part of the
 *    library's code object, not allocated at run time).
 *  - Streams: GPU work is enqueued on the HIP stream passed as `stream`
 *    (a hipStream_t; NULL means the default stream) and the call returns
 *    without synchronising.  A fault inside a kernel surfaces at the caller's
 *    next synchronisation, as for any HIP launch.
 *  - Heads: tensor head h (0-based) uses a[h], b[h], w[h]; the usual choice
 *    is Wythoff row h + 1 (fibatt_wythoff).  Requirements: a[h] >= 0,
 *    b[h] >= 1 (so the sequence grows and (0, 0) is impossible),
 *    1 <= w[h] <= N.  A distance of 0 (a[h] = 0) is the diagonal and counts
 *    once.  Distances >= N have no pairs.
 */
#ifndef FIBATT_H
#define FIBATT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FIBATT_OK = 0,
  FIBATT_E_INVAL = 1,       /* bad argument: null pointer, bad size, bad a/b/w, misalignment */
  FIBATT_E_RANGE = 2,       /* a result does not fit the caller's buffer or int32 */
  FIBATT_E_UNSUPPORTED = 3, /* valid but not implemented: d_h, dtype, H above FIBATT_MAX_HEADS */
  FIBATT_E_HIP = 4          /* the HIP runtime reported an error while enqueuing work */
} fibatt_status;

typedef enum {
  FIBATT_F32 = 0,  /* IEEE binary32 */
  FIBATT_BF16 = 1  /* bfloat16 */
} fibatt_dtype;

/* Largest number of heads one call accepts. */
#define FIBATT_MAX_HEADS 128

/* Problem description shared by fibatt_fwd and fibatt_bwd.
 *  B, H, N, d_h : batch, heads, tokens per sequence, head width (64 or 128).
 *  dtype        : element type of Q, K, V, O and dO (a fibatt_dtype value).
 *  a, b, w      : HOST arrays of H int32 each (see "Heads" above); read
 *                 during the call only. */
typedef struct {
  int32_t B, H, N, d_h;
  int32_t dtype;
  const int32_t* a;
  const int32_t* b;
  const int32_t* w;
} fibatt_desc;

/* Row i >= 1 of the Wythoff array: *a = floor(floor(i*phi)*phi),
 * *b = floor(floor(i*phi)*phi^2) = *a + floor(i*phi), computed in exact
 * integer arithmetic.  The Fibottention paper (Wythoff array paragraph) takes
 * head i's sequence from this row, whose rows are disjoint and cover every
 * positive integer.  Errors: E_INVAL if i < 1 or a pointer is NULL, E_RANGE
 * if *b would exceed INT32_MAX. */
int fibatt_wythoff(int32_t i, int32_t* a, int32_t* b);

/* The modified pair of README Algorithm 2 (its is_modified branch) for
 * Wythoff row i >= 1: with (a, b) = fibatt_wythoff(i), *b = b - a and
 * *a = a - (b - a), the Fibonacci recurrence run two steps back, so that
 * Fib(*a, *b) = *a, *b, a, b, ...  For row 1 this is (0, 1): head 1 then
 * attends distance 0 as well.  Computed as its closed form
 * (i - 1, floor(i*phi)) in exact integers.  Errors: E_INVAL if i < 1 or a
 * pointer is NULL, E_RANGE if floor(i*phi) would exceed INT32_MAX. */
int fibatt_wythoff_modified(int32_t i, int32_t* a, int32_t* b);

/* Per-head windows interpolated between w_min and w_max (Fibottention paper,
 * method section): w[i - 1] = w_min + floor((w_max - w_min)(i - 1)/(H - 1))
 * for heads i = 1..H; a single head gets w_max (the formula is undefined
 * for H = 1).  w is a host array of H int32.  Errors: E_INVAL for H < 1,
 * w NULL, w_min < 1 or w_max < w_min. */
int fibatt_windows(int32_t H, int32_t w_min, int32_t w_max, int32_t* w);

/* Host-only offset table (no GPU involved).  For each head h, the distinct
 * distances f of Fib(a[h], b[h]) with f <= min(w[h], N - 1), ascending
 * (README Algorithm 1 generates the sequence; the paper's set definition
 * keeps the terms within the window).  Output in CSR form:
 *   head_ptr[H + 1] : head_ptr[0] = 0, head h owns offs[head_ptr[h] .. head_ptr[h+1]).
 *   offs[offs_cap]  : the distances (int32).
 * head_ptr is always written in full on success or E_RANGE.  If the total
 * exceeds offs_cap the call returns E_RANGE, writes only head_ptr, and
 * head_ptr[H] is the capacity needed (two-call sizing).  offs may be NULL
 * when offs_cap is 0.  Errors: E_INVAL for H < 1, N < 1, NULL arrays or bad
 * a/b/w. */
int fibatt_offsets(int32_t H, int32_t N, const int32_t* a, const int32_t* b,
                   const int32_t* w, int32_t* head_ptr, int32_t* offs,
                   int32_t offs_cap);

/* Forward pass.  Device pointers:
 *   q, k, v : [B, H, N, d_h] in desc->dtype (read).
 *   o       : [B, H, N, d_h] in desc->dtype (written): O_j = sum_k P_jk V_k.
 *   lse     : [B, H, N] fp32 (written): natural-log log-sum-exp of row j's
 *             scaled scores; -inf for a row with no key in its support, whose
 *             O row is then 0.
 * Accumulation is fp32 for either dtype.  Errors: E_INVAL, E_UNSUPPORTED
 * (d_h not 64/128, dtype not F32/BF16, H > FIBATT_MAX_HEADS), E_HIP. */
int fibatt_fwd(const fibatt_desc* desc, const void* q, const void* k,
               const void* v, void* o, float* lse, void* stream);

/* Number of fp32 elements of the workspace fibatt_bwd needs (B*H*N), or -1
 * for an invalid descriptor. */
int64_t fibatt_bwd_workspace_floats(const fibatt_desc* desc);

/* Backward pass: gradients of sum(O * dO) for the forward above.
 *   q, k, v, dout : [B, H, N, d_h] in desc->dtype (read).
 *   lse           : [B, H, N] fp32 (read): what fibatt_fwd produced for the
 *                   same q, k, v.  The forward output O itself is not needed.
 *   dq, dk, dv    : [B, H, N, d_h] fp32 (written).
 *   workspace     : fibatt_bwd_workspace_floats(desc) fp32 elements of device
 *                   scratch (contents on entry ignored, clobbered).
 * With P the support-restricted softmax (recomputed from lse),
 * dP_jk = dO_j . V_k and D_j = sum_k P_jk dP_jk (summed in fp32, which is
 * dO_j . O_j without O's storage rounding): dS = P (dP - D),
 * dQ = dS K / sqrt(d_h), dK = dS^T Q / sqrt(d_h), dV = P^T dO.  The support
 * is symmetric, so dK and dV are gathered key by key over the same offsets
 * (no atomics; results are bitwise reproducible run to run).  Errors as for
 * fibatt_fwd. */
int fibatt_bwd(const fibatt_desc* desc, const void* q, const void* k,
               const void* v, const float* lse, const void* dout, float* dq,
               float* dk, float* dv, float* workspace, void* stream);

/* Class-token variant (README Algorithm 2's mask over a class token and N
 * patches: all ones, with the head's Fibonacci pattern among the patches).
 * Token 0 is the class token: row 0 attends every key, every row attends
 * key 0, and among tokens 1..N-1 the support is the head's as above (the
 * distance between two patches is the same as between their positions).
 * Pair (0, 0) is in the support.  Every row therefore has at least one key:
 * LSE is finite everywhere.  Same layouts, ownership and error behaviour as
 * fibatt_fwd / fibatt_bwd.  Row 0 and column 0 are dense reductions over the
 * slab done in fixed order (bitwise reproducible): inside the bf16 d_h = 64
 * kernels for N <= 240 (forward) and N <= 201 (backward), by separate dense
 * row/column kernels otherwise.
 *
 * Workspace: fibatt_fwd_cls_workspace_floats(desc) fp32 elements (0 when N
 * <= 1024, and then `workspace` may be NULL), fibatt_bwd_cls_workspace_floats
 * (desc) for the backward (B*H*(N + d_h) + d_h, plus partial sums when
 * N > 1024).  Both
 * return -1 for an invalid descriptor.  Contents on entry are ignored. */
int64_t fibatt_fwd_cls_workspace_floats(const fibatt_desc* desc);
int64_t fibatt_bwd_cls_workspace_floats(const fibatt_desc* desc);

/* Forward with the class-token mask.  Arguments as fibatt_fwd, plus the
 * workspace described above. */
int fibatt_fwd_cls(const fibatt_desc* desc, const void* q, const void* k,
                   const void* v, void* o, float* lse, float* workspace,
                   void* stream);

/* Backward with the class-token mask: gradients of sum(O * dO) for
 * fibatt_fwd_cls.  Arguments as fibatt_bwd (lse must come from
 * fibatt_fwd_cls); workspace as described above. */
int fibatt_bwd_cls(const fibatt_desc* desc, const void* q, const void* k,
                   const void* v, const float* lse, const void* dout, float* dq,
                   float* dk, float* dv, float* workspace, void* stream);

/* Heads given by an explicit distance table instead of (a, b, w): any
 * symmetric dilation set, e.g. the constant-factor (c n) and exponential
 * dilation sequences that the Fibottention paper's method section sets its
 * Fibonacci sequences against (support set of a general sequence (f_n) and
 * window w), or a table from fibatt_offsets edited by hand.  Query
 * j attends key k iff |j - k| is one of its head's distances (0 is the
 * diagonal); everything else is as for fibatt_fwd / fibatt_bwd (or, with
 * cls = 1, as for fibatt_fwd_cls / fibatt_bwd_cls).
 *  head_ptr    : HOST, H + 1 int32, head_ptr[0] = 0, non-decreasing; head h
 *                owns entries head_ptr[h] .. head_ptr[h + 1] - 1, at most 64.
 *  offs        : HOST, head_ptr[H] int32 distances, strictly ascending within
 *                a head, each in [0, N - 1] (checked on the host).
 *  offs_device : DEVICE copy of offs (same values, 4-byte aligned), read by
 *                the kernels; it must stay valid until the enqueued work has
 *                run.  The library cannot check that it equals offs.
 * Errors: as fibatt_fwd, plus E_INVAL for a malformed table and
 * E_UNSUPPORTED for a head with more than 64 distances. */
typedef struct {
  int32_t B, H, N, d_h;
  int32_t dtype;
  int32_t cls; /* 0: mask from the table only; 1: plus the class-token row and column */
  const int32_t* head_ptr;
  const int32_t* offs;
  const int32_t* offs_device;
} fibatt_table_desc;

/* Workspace sizes (fp32 elements) for the two calls below, or -1 for an
 * invalid descriptor: forward 0 (cls = 0) or as fibatt_fwd_cls_workspace_floats;
 * backward B*H*N (cls = 0) or as fibatt_bwd_cls_workspace_floats. */
int64_t fibatt_fwd_table_workspace_floats(const fibatt_table_desc* desc);
int64_t fibatt_bwd_table_workspace_floats(const fibatt_table_desc* desc);

/* Forward and backward with table heads; arguments as fibatt_fwd_cls /
 * fibatt_bwd_cls (the forward workspace may be NULL when its size is 0). */
int fibatt_fwd_table(const fibatt_table_desc* desc, const void* q,
                     const void* k, const void* v, void* o, float* lse,
                     float* workspace, void* stream);
int fibatt_bwd_table(const fibatt_table_desc* desc, const void* q,
                     const void* k, const void* v, const float* lse,
                     const void* dout, float* dq, float* dk, float* dv,
                     float* workspace, void* stream);

/* Strided tensors.  Row n of head h of batch b of a tensor starts at
 * element b*sb + h*sh + n*sn of its buffer (strides in elements of that
 * tensor's own type); the row's d_h elements are contiguous.  The dense
 * [B, H, N, d_h] layout is {H*N*d_h, N*d_h, d_h}; the Q of a fused QKV
 * projection stored [B, N, 3, H, d_h] is {3*N*H*d_h, d_h, 3*H*d_h} at
 * offset 0 (K at H*d_h, V at 2*H*d_h), and an output in [B, N, H, d_h]
 * (ready for the output projection) is {N*H*d_h, d_h, H*d_h}.
 * Requirements, checked on the host: strides >= 0, sn >= d_h, every stride
 * times the element size a multiple of 16 bytes (with 16-byte aligned base
 * pointers every row is then 16-byte aligned), and the largest element
 * offset below 2^62.  Not checkable and left to the caller: the buffers hold
 * every row, and distinct rows of an output do not overlap each other or
 * any input.  LSE and the workspace stay dense [B, H, N]. */
typedef struct {
  int64_t sb, sh, sn;
} fibatt_layout;

/* Layouts of one call's tensors; the forward reads q, k, v, o and ignores
 * the rest, the backward ignores o. */
typedef struct {
  fibatt_layout q, k, v, o, dout, dq, dk, dv;
} fibatt_layouts;

/* Forward and backward with strided tensors: otherwise as fibatt_fwd /
 * fibatt_bwd (cls = 0) or fibatt_fwd_cls / fibatt_bwd_cls (cls = 1).
 * Workspaces (fp32 elements): forward none with cls = 0 (may be NULL),
 * fibatt_fwd_cls_workspace_floats(desc) with cls = 1 (0, and then NULL is
 * allowed, for N <= 1024); backward fibatt_bwd_workspace_floats(desc)
 * (cls = 0) or fibatt_bwd_cls_workspace_floats(desc) (cls = 1).  Every
 * kernel family reads and writes strided rows; the kernels chosen are the
 * same as for dense tensors of that shape.  Errors: as fibatt_fwd, plus
 * E_INVAL for a bad layout or cls not 0/1. */
int fibatt_fwd_strided(const fibatt_desc* desc, int32_t cls,
                       const fibatt_layouts* layouts, const void* q,
                       const void* k, const void* v, void* o, float* lse,
                       float* workspace, void* stream);
int fibatt_bwd_strided(const fibatt_desc* desc, int32_t cls,
                       const fibatt_layouts* layouts, const void* q,
                       const void* k, const void* v, const float* lse,
                       const void* dout, float* dq, float* dk, float* dv,
                       float* workspace, void* stream);

/* Backward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, layouts, results and error
 * behaviour as fibatt_bwd, minus `workspace`: the kernels' scratch (D per
 * row) is a fixed array of FIBATT_NOALLOC_MAX_ROWS floats (16 MiB) in the
 * library's device memory, one copy per GPU, held until the process ends.
 * The call allocates nothing.
 *  - B*H*N above FIBATT_NOALLOC_MAX_ROWS: FIBATT_E_RANGE, nothing enqueued.
 *  - Every call on one GPU uses that GPU's single array (its contents on
 *    entry are ignored and left clobbered): calls that overlap on one GPU,
 *    i.e. run concurrently on different streams, race and give undefined
 *    results; calls ordered on one stream are safe. */
#define FIBATT_NOALLOC_MAX_ROWS (1 << 22)
int fibatt_bwd_noalloc(const fibatt_desc* desc, const void* q, const void* k,
                       const void* v, const float* lse, const void* dout,
                       float* dq, float* dk, float* dv, void* stream);

/* Measurement aids (not part of the attention itself). */

/* Binds two HIP events (hipEvent_t values created by the caller) to the GPU
 * execution of the next call on this thread that enqueues work: start_event
 * to the start of its first kernel, stop_event to the end of its last
 * kernel, both recorded by the GPU around the kernels themselves
 * (hipExtLaunchKernelGGL).  hipEventElapsedTime(start, stop) is then the
 * time of that call's kernels without the launch gaps around them (the
 * kernel durations a profiler reports).  The binding is used by that one
 * call and then cleared, also when the call fails; passing NULL for both
 * clears it.  Errors: E_INVAL if exactly one event is NULL. */
int fibatt_time_next_call(void* start_event, void* stop_event);

/* The HBM traffic of a pass with nothing else in it, as a reference for the
 * bandwidth the GPU delivers at that read/write mix: reads n_src device
 * arrays of `bytes` each and writes n_dst device arrays of
 * dst_scale * `bytes` each (16-byte units, coalesced; every unit written is
 * the xor of the units read).  The forward of bf16 inputs has the mix
 * n_src = 3, n_dst = 1, dst_scale = 1 (Q, K, V read, O written); its
 * backward n_src = 4, n_dst = 3, dst_scale = 2 (Q, K, V, dO read; fp32 dQ,
 * dK, dV written).  src and dst are HOST arrays of device pointers (16-byte
 * aligned).  Errors: E_INVAL for counts outside 1..4, dst_scale not 1 or 2,
 * bytes not a positive multiple of 16, NULL or misaligned pointers; E_HIP. */
int fibatt_hbm_stream(const void* const* src, int32_t n_src, void* const* dst,
                      int32_t n_dst, int64_t bytes, int32_t dst_scale,
                      void* stream);

/* The rate at which the XCDs' L2 caches fill from beyond them, as a
 * reference for kernels whose L2 misses bound them: every one of the 8 XCDs
 * reads the whole device buffer buf (`bytes`, a multiple of 4 MiB), `passes`
 * times; a buffer larger than one XCD's L2 (4 MiB) misses there on every
 * read.  The bytes delivered to the CUs are 8 * bytes * passes.  out is a
 * device array of FIBATT_FABRIC_OUT_BYTES that receives one 16-byte xor of
 * the data per workgroup (so no read can be dropped).  Errors: E_INVAL for
 * bytes not a positive multiple of 4 MiB, passes < 1, NULL or misaligned
 * pointers; E_HIP. */
#define FIBATT_FABRIC_OUT_BYTES (16 * 8 * 128)
int fibatt_fabric_read(const void* buf, int64_t bytes, int32_t passes, void* out,
                       void* stream);

/* Message describing the last error on the calling thread ("" if none).
 * The pointer stays valid until the thread's next fibatt_* call. */
const char* fibatt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FIBATT_H */
