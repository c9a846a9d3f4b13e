/*
 * kvstore.h -- C ABI of the MI355X (gfx950) paged varlen attention library.
 *
 * Two operations, both from the step list of one decoder layer in
 * "Transformer 추론 커널: GEMM·Attention·FlashAttention·Fusion (3/10)", §2:
 * the KV-cache store that precedes attention, and attention of the new query
 * rows against the paged K/V.  Everything else is plumbing for those two.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors travel as borrowed descriptors (kvs_tensor): a data pointer plus
 *    dtype, rank, shape and strides in ELEMENTS.  The library never copies,
 *    frees or retains them.  Every tensor must be dense row-major
 *    (stride[ndim-1] == 1, stride[i] == stride[i+1] * shape[i+1]) and its data
 *    pointer 16-byte aligned.
 *  - Every data pointer is a DEVICE pointer on the current HIP device, owned by
 *    the caller, except where a comment says "host".
 *  - Calls are asynchronous on `stream`: they validate on the host, enqueue
 *    kernels (and, for the plain attn_varlen_paged, stream-ordered allocations
 *    on `stream`), and return.  No call reads device memory from the host, and
 *    none synchronises the device except kvs_release_workspace (a teardown
 *    call) and the calls of the debug library below.
 *  - The paged pool (k_cache, v_cache) is [num_blocks, 16, Hkv, D]: token row
 *    `r` of physical block `p` holds the K (or V) vectors of all Hkv heads.  A
 *    slot number names one token row: slot = p * 16 + r.  Page size 16 follows
 *    "tiny-vLLM: CUDA로 직접 쓴 LLM 추론 엔진 읽기", entry 6; page = slot // 16 and
 *    row = slot % 16 follow the token-granular table of "장부가 커널 인자로 바뀌는
 *    지점과 CUDA graph", section "장부에서 텐서로".
 *  - Errors: a non-zero kvs_status means nothing was enqueued (except
 *    KVS_ERR_HIP, where a launch was attempted).  kvs_last_error() returns the
 *    calling thread's message for its last non-OK status.
 *  - Values that live on the device (lengths, table entries, slots) cannot be
 *    checked without a synchronisation; the preconditions stated below for them
 *    are the caller's responsibility, and violating them is undefined behaviour
 *    (out-of-range table entries or slots are out-of-bounds device accesses).
 *  - Debug library (libkvstore_debug.so: the same kernels, this ABI built with
 *    KVS_DEBUG): every call first checks those values on the GPU --
 *    cu_seqlens_q[0] = 0 and cu_seqlens_q[B] = T, 1 <= Lq_b <= Lk_b <= 16 MB,
 *    each block-table entry the call reads in [0, NB), each store slot below
 *    16 NB -- waits for the check, and on a violation returns KVS_ERR_INVALID
 *    naming it with nothing else enqueued.  It synchronises the stream, so it
 *    cannot be captured into a graph.
 */
#ifndef KVSTORE_H
#define KVSTORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* kvs_stream_t; /* a hipStream_t; NULL = the null stream */

typedef enum {
  KVS_OK = 0,
  KVS_ERR_INVALID = 1,      /* bad argument: null pointer, shape/dtype/stride mismatch   */
  KVS_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head dim, page size, group) */
  KVS_ERR_WORKSPACE = 3,    /* caller workspace too small                                */
  KVS_ERR_HIP = 4           /* a HIP runtime call or launch failed                       */
} kvs_status;

typedef enum { KVS_F32 = 0, KVS_BF16 = 1, KVS_I32 = 2, KVS_FP8_E4M3 = 3, KVS_INT8 = 4 } kvs_dtype;   /* FP8: OCP E4M3 codes; INT8: signed codes; 1 byte each */

typedef struct {
  void* data;          /* device pointer (16-byte aligned)                 */
  int32_t dtype;       /* kvs_dtype                                        */
  int32_t ndim;        /* 1..4                                             */
  int64_t shape[4];
  int64_t stride[4];   /* in elements; must describe a dense row-major view */
} kvs_tensor;

/*
 * kv_store_paged -- write new K/V token rows into their slots.
 *
 * Defined by the store step that comes right before attention ("Transformer 추론
 * 커널 (3/10)", §2) and by the decode path appending the new token's K/V to the
 * paged cache ("tiny-vLLM ...", entry 5).
 *
 *   k_new, v_new   [T_new, Hkv, D], dtype f32 or bf16 (same as the caches)
 *   slot_mapping   i32 [T_new]; row t goes to slot slot_mapping[t];
 *                  a negative slot skips the row (a padding row owns no slot)
 *   k_cache,v_cache [NB, 16, Hkv, D], written in place
 *
 * Preconditions on device values: every non-negative slot < 16 * NB, and no two
 * rows name the same slot (duplicates leave either row's data, unspecified).
 * The copy is bit-exact.  T_new == 0 is a valid no-op.
 */
kvs_status kv_store_paged(const kvs_tensor* k_new, const kvs_tensor* v_new,
                          const kvs_tensor* slot_mapping,
                          kvs_tensor* k_cache, kvs_tensor* v_cache,
                          kvs_stream_t stream);

/* Layout of the rotary pairs of a head (kv_store_rope_paged). */
typedef enum { KVS_ROPE_NEOX = 0, KVS_ROPE_INTERLEAVED = 1 } kvs_rope_style;

typedef struct {
  int32_t rotary_dim;  /* dims rotated per head: a multiple of 16 in [16, D]; 0 = D   */
  int32_t style;       /* kvs_rope_style: pairs (i, i + rotary_dim/2) or (2i, 2i + 1) */
  double base;         /* theta_i = base^(-2 i / rotary_dim); finite, > 0             */
  double pos_scale;    /* angle = (position / pos_scale) * theta_i; finite, > 0       */
} kvs_rope;

/*
 * kv_store_rope_paged -- the "RoPE + KV cache store" step in one pass: rotate
 * q in place, and write the rotated k_new and the unchanged v_new into their
 * slots.
 *
 * A layer's step list applies a rotary position embedding to Q and K right
 * before attention, fused with the KV-cache write ("Transformer 추론 커널 (3/10)",
 * §1-§2); its variant, scaling and offset are dispatch and test axes (§19,
 * §24).  The pages give no formula; the rotation is RoFormer's (Su et al.
 * 2021, section 3.2): pair i of token t is turned by
 *   a = (positions[t] / pos_scale) * base^(-2 i / rotary_dim),
 *   x1' = x1 cos a - x2 sin a,   x2' = x2 cos a + x1 sin a,
 * with the pairs of `style`; dims at or past rotary_dim are unchanged.
 * Angles are formed in double precision; the rotation runs in fp32 and the
 * result is rounded to the tensor dtype (nearest even for bf16).
 *
 *   q            [T, Hq, D] f32 or bf16, rotated in place; NULL = no query rows
 *   k_new, v_new [T, Hkv, D] same dtype (read only)
 *   positions    i32 [T]: token t's position (any offset is the caller's)
 *   slot_mapping i32 [T]: pool slot of row t; negative = not stored (q row t
 *                is still rotated)
 *   k_cache, v_cache [NB, 16, Hkv, D]: slot s is written with row t's rotated
 *                K and its V
 *   rope         rotation parameters (host memory, read during the call)
 * Supported: D a multiple of 16 up to 256, page size 16.  Preconditions on
 * device values: no two rows name the same slot; slots >= 16 * NB are skipped.
 * T == 0 is a no-op.  Allocates nothing.
 */
kvs_status kv_store_rope_paged(kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                               const kvs_tensor* positions, const kvs_tensor* slot_mapping,
                               kvs_tensor* k_cache, kvs_tensor* v_cache, const kvs_rope* rope,
                               kvs_stream_t stream);

/*
 * attn_varlen_paged -- exact softmax attention of packed varlen query rows over
 * a paged K/V cache.
 *
 * Computes, for every sequence b, new row i and query head h,
 *     out[t, h, :] = sum_j softmax_j(scale * q[t, h, :] . K_b[j, g, :]) V_b[j, g, :]
 *     lse[t, h]    = ln sum_j exp(scale * q[t, h, :] . K_b[j, g, :])
 * over the visible keys j, where t = cu_seqlens_q[b] + i, g = h / (Hq / Hkv)
 * (several query heads share one KV head: "Transformer 추론 커널 (3/10)", §15),
 * and K_b[j] is row j % 16 of physical block block_table[b, j / 16] (§14).
 * The formula is the scaled dot-product attention of §10; it is computed as a
 * tiled pass with online softmax (§11, §12), which reaches the same exact result
 * without materialising the score matrix.
 *
 * Visible keys: with Lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] new rows and
 * Lk_b = seqlens_k[b] keys in total, the cached prefix is c_b = Lk_b - Lq_b and
 * row i sits at position c_b + i.  If `causal` and Lq_b > 1, row i sees keys
 * 0 .. c_b + i; otherwise it sees all Lk_b keys.  (Query length = extend length,
 * key length = the whole length so far, as in "장부가 커널 인자로 바뀌는 지점과 CUDA
 * graph", section "장부에서 텐서로".)
 *
 *   q            [T, Hq, D]  f32 or bf16, T = total new rows
 *   k_cache/v_cache [NB, 16, Hkv, D], same dtype as q
 *   block_table  i32 [B, MB]; only entries 0 .. ceil(Lk_b/16)-1 of row b are read
 *   cu_seqlens_q i32 [B+1]
 *   seqlens_k    i32 [B]
 *   scale        multiplies q.k before the mask and softmax (1/sqrt(D) usually)
 *   out          [T, Hq, D]  same dtype as q (rounded to nearest even for bf16)
 *   lse          f32 [T, Hq], or NULL to skip it
 *
 * Supported: D in {64, 128}; page size 16; Hq % Hkv == 0; for the decode path
 * Hq / Hkv <= 16.  Anything else returns KVS_ERR_UNSUPPORTED -- there is no
 * slower fallback path.
 * Preconditions on device values: cu_seqlens_q[0] == 0, cu_seqlens_q[B] == T,
 * 1 <= Lq_b <= Lk_b <= 16 * MB, and every table entry that is read lies in
 * [0, NB).  Tail rows of a sequence's last block and entries past its last block
 * are never used (their contents do not matter).
 * Dispatch uses shapes only: T == B (one new row per sequence) takes the decode
 * path; otherwise the prefill/extend path.  The decode path cuts the batch's
 * key blocks into equal ranges (split-KV, "Transformer 추론 커널 (3/10)", §16)
 * and needs scratch memory for the pieces of split sequences (§16: partial
 * results of the pieces, merged afterwards): this call keeps one grow-only
 * device buffer per device for it.  When a call needs more than the buffer
 * holds, a new one is allocated stream-ordered on `stream` (hipMallocAsync),
 * zeroed there by the library's own kernel, and the old one freed
 * stream-ordered on `stream`; nothing synchronises the device.
 * kvs_release_workspace frees it.  Calls on one device that overlap in time
 * (different streams with no ordering between them) share that buffer and are
 * not allowed; use attn_varlen_paged_ex with separate workspaces for that.  A
 * call that grows the buffer while its stream is captured into a graph
 * records the allocation in the graph: capture _ex calls instead.
 */
kvs_status attn_varlen_paged(const kvs_tensor* q,
                             const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                             const kvs_tensor* block_table,
                             const kvs_tensor* cu_seqlens_q,
                             const kvs_tensor* seqlens_k,
                             float scale, int causal,
                             kvs_tensor* out, kvs_tensor* lse,
                             kvs_stream_t stream);

/*
 * attn_varlen_paged_noalloc -- attn_varlen_paged for callers that cannot
 * allocate memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, computation, paths and
 * results as attn_varlen_paged (the same kernels); it allocates nothing, on
 * the device or the host.  The split decode's scratch is a static device
 * array of 16 MiB inside the library (one per GPU the library runs on, held
 * until the process ends); shapes whose split plan needs more return
 * KVS_ERR_WORKSPACE with nothing enqueued (attn_varlen_paged_workspace_size
 * with NULL hints gives the need).  Each call first clears the merge counters
 * it uses with one of the library's kernels on `stream`.  Every call on a GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (on
 * different streams with no ordering between them) race and are not allowed.
 */
kvs_status attn_varlen_paged_noalloc(const kvs_tensor* q,
                                     const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                     const kvs_tensor* block_table,
                                     const kvs_tensor* cu_seqlens_q,
                                     const kvs_tensor* seqlens_k,
                                     float scale, int causal,
                                     kvs_tensor* out, kvs_tensor* lse,
                                     kvs_stream_t stream);

/* Optional host-side hints for attn_varlen_paged_ex; 0 means "unknown / choose".
 * The kernel-facing bookkeeping of "장부가 커널 인자로 바뀌는 지점과 CUDA graph"
 * ("장부에서 텐서로") carries host-side max_seqlen_q / max_seqlen_k next to the
 * device tensors; num_splits is the split-KV degree of "Transformer 추론 커널
 * (3/10)", §16; decode_tail states the phase order of a mixed batch (§6). */
typedef struct {
  int32_t max_seqlen_q;  /* upper bound on Lq_b (host value), 0 = unknown; unused now  */
  int32_t max_seqlen_k;  /* upper bound on Lk_b (host value), 0 = unknown; unused now  */
  int32_t num_splits;    /* decode: number of equal ranges the batch's key blocks are
                            cut into (one workgroup each); 0 = automatic.  Raised
                            if needed so a range holds at most 2048 blocks.       */
  int32_t decode_tail;   /* N > 0: the caller states that the last N sequences of the
                            batch have one query row each (a mixed serving batch with
                            its decode rows last, as a scheduler forms it).  Sequences
                            [0, B - N) then take the prefill/extend path and the last
                            N the decode path, two launches on the same stream, which
                            spreads the decode rows' contexts over the whole device
                            instead of one work item each.  A wrong statement gives
                            wrong rows for the sequences it misdescribes (every access
                            stays inside the given buffers).  N = B needs T == B.
                            Ignored (one launch) when an lse row view would not be
                            16-byte aligned.  Only the decode part uses the workspace;
                            pass the same hints to attn_varlen_paged_workspace_size. */
} kvs_hints;

/* Bytes of device scratch attn_varlen_paged_ex needs for these shapes and hints
 * (0 when the chosen path needs none): the partial results and merge counters
 * of a split decode ("Transformer 추론 커널 (3/10)", §16: more pieces mean more
 * parallelism but a partial buffer and a reduction).  `hints` (may be NULL)
 * must be the ones the call will get.  Returns (size_t)-1 on invalid shapes. */
size_t attn_varlen_paged_workspace_size(const kvs_tensor* q, const kvs_tensor* k_cache,
                                        const kvs_tensor* block_table,
                                        const kvs_hints* hints);

/*
 * attn_varlen_paged_ex -- attn_varlen_paged with caller-owned scratch and hints.
 * Same computation and argument meaning; the scratch holds the split-KV pieces
 * of "Transformer 추론 커널 (3/10)", §16.  `workspace` is a device buffer of at
 * least attn_varlen_paged_workspace_size(q, k_cache, block_table, hints) bytes,
 * 256-byte aligned (may be NULL when that size is 0).  It must be zero-filled
 * before its first use with this library.  Its first 4 MiB hold the split
 * decode's per-(sequence, KV head) counters at a place that does not depend on
 * the shapes, and every call leaves them at zero, so one workspace, zeroed
 * once, serves any sequence of calls of any shapes (each needing no more than
 * its size).  Two calls that overlap in time must not share it.  Allocates
 * nothing.  `hints` may be NULL.  A split decode (more than one range) needs
 * B * Hkv <= 2^20, else KVS_ERR_UNSUPPORTED.
 */
kvs_status attn_varlen_paged_ex(const kvs_tensor* q,
                                const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                const kvs_tensor* block_table,
                                const kvs_tensor* cu_seqlens_q,
                                const kvs_tensor* seqlens_k,
                                float scale, int causal,
                                kvs_tensor* out, kvs_tensor* lse,
                                const kvs_hints* hints,
                                void* workspace, size_t workspace_bytes,
                                kvs_stream_t stream);

/*
 * attn_decode_append_paged -- one decode step in one launch: each sequence's
 * new key/value row is appended to the cache and the sequence's query row
 * attends over all of its keys, the new one included.
 *
 * The result, in `out`, `lse` and the caches, is that of
 *   kv_store_paged(k_new, v_new, slots, k_cache, v_cache)   with
 *     slots[b] = block_table[b][(Lk_b - 1) / 16] * 16 + (Lk_b - 1) % 16,
 *   then attn_varlen_paged_ex(q, ..., cu_seqlens_q = {0, 1, .., B}, seqlens_k,
 *     scale, causal = 1, out, lse, hints, workspace, ...)
 * -- store before attention ("Transformer 추론 커널 (3/10)", §2), with the new
 * token's K/V as key Lk_b - 1 (decode adds one token per sequence to the paged
 * cache: "tiny-vLLM ...", entry 5).  The
 * launch reads the new row from k_new / v_new rather than from the cache, so
 * the store and the attention need no ordering between them.
 *
 *   q            [B, Hq, D]  f32 or bf16, one query row per sequence
 *   k_new/v_new  [B, Hkv, D] same dtype; row b is sequence b's new token
 *   k_cache/v_cache [NB, 16, Hkv, D]; the slot of key Lk_b - 1 is written
 *   block_table  i32 [B, MB];  seqlens_k  i32 [B] (Lk_b counts the new token)
 *   out, lse, hints, workspace: as for attn_varlen_paged_ex (the workspace
 *     size is attn_varlen_paged_workspace_size(q, k_cache, block_table, hints))
 * Preconditions on device values: 1 <= Lk_b <= 16 * MB and every table entry
 * that is read lies in [0, NB); the slots of different sequences differ, and
 * no sequence reads, as one of its keys, a slot that another sequence's new
 * row is written to (as with the two separate calls, whose order would decide
 * what such a read sees).
 * Same support limits and errors as the decode path of attn_varlen_paged.
 * Allocates nothing.
 */
kvs_status attn_decode_append_paged(const kvs_tensor* q,
                                    const kvs_tensor* k_new, const kvs_tensor* v_new,
                                    kvs_tensor* k_cache, kvs_tensor* v_cache,
                                    const kvs_tensor* block_table,
                                    const kvs_tensor* seqlens_k,
                                    float scale,
                                    kvs_tensor* out, kvs_tensor* lse,
                                    const kvs_hints* hints,
                                    void* workspace, size_t workspace_bytes,
                                    kvs_stream_t stream);

/*
 * attn_varlen_paged_window_ex -- attn_varlen_paged_ex with a sliding-window
 * causal mask.  The pages list the sliding window among the masks a kernel
 * dispatch has to cover and a test matrix has to exercise ("Transformer 추론
 * 커널 (3/10)", §19 and §24); the band taken here is the usual one: with
 * window W the row at position p (the causal position c_b + i, so a one-row
 * decode sits at Lk_b - 1) sees keys max(0, p - W + 1) .. p -- its own and the
 * W - 1 before it.  Same arguments as attn_varlen_paged_ex with `causal`
 * replaced by `window` (W >= 1, else KVS_ERR_INVALID); same paths, limits,
 * workspace and errors.  Keys below the first row's window start in a
 * sequence, and the block-table entries of blocks holding only such keys, are
 * never read (a caller may have freed those blocks).
 */
kvs_status attn_varlen_paged_window_ex(const kvs_tensor* q,
                                       const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                       const kvs_tensor* block_table,
                                       const kvs_tensor* cu_seqlens_q,
                                       const kvs_tensor* seqlens_k,
                                       float scale, int32_t window,
                                       kvs_tensor* out, kvs_tensor* lse,
                                       const kvs_hints* hints,
                                       void* workspace, size_t workspace_bytes,
                                       kvs_stream_t stream);

/*
 * attn_decode_append_paged_window -- attn_decode_append_paged with the
 * sliding window of attn_varlen_paged_window_ex (the mask variant of
 * "Transformer 추론 커널 (3/10)", §19 and §24): sequence b's query row sees
 * keys max(0, Lk_b - W) .. Lk_b - 1, the new one included.  Same result as
 * kv_store_paged then attn_varlen_paged_window_ex with cu_seqlens_q = 0..B.
 * W >= 1, else KVS_ERR_INVALID.  Table entries below block
 * max(0, Lk_b - W) / 16 are never read.
 */
kvs_status attn_decode_append_paged_window(const kvs_tensor* q,
                                           const kvs_tensor* k_new, const kvs_tensor* v_new,
                                           kvs_tensor* k_cache, kvs_tensor* v_cache,
                                           const kvs_tensor* block_table,
                                           const kvs_tensor* seqlens_k,
                                           float scale, int32_t window,
                                           kvs_tensor* out, kvs_tensor* lse,
                                           const kvs_hints* hints,
                                           void* workspace, size_t workspace_bytes,
                                           kvs_stream_t stream);

/*
 * FP8 KV cache.  The pages list FP8 and INT8 KV, and quantized KV layouts,
 * among the dtypes and layouts a kernel dispatch covers ("Transformer 추론 커널
 * (3/10)", §19) and quantized KV in the edge-case matrix (§24), and ask that the
 * quantization group and scale layout be what the kernel expects (§7); they
 * fix no format.  Here: codes in the OCP E4M3 format (bias 7, subnormal step
 * 2^-9, largest finite 448, no infinities); the D values of one token row of
 * one KV head share one fp32 scale s; the value of a code c is E4M3(c) * s.
 *
 *   k_cache, v_cache [NB, 16, Hkv, D] dtype KVS_FP8_E4M3 (codes)
 *   k_scale, v_scale [NB, Hkv, 16] f32: scale of (block, head, row); a head's
 *                    16 rows of a block are contiguous
 */

/*
 * kv_store_paged_fp8 -- quantize new K/V token rows and write them into their
 * slots (the KV-cache store of "Transformer 추론 커널 (3/10)", §2, into the FP8
 * layout of §19; the scale layout follows §7): for each row t and KV head h, s = absmax_d |x[t, h, d]| / 448 (0 for an
 * all-zero row) and code[d] = the E4M3 value nearest to x / s (ties to even,
 * saturated at +-448), both divisions in fp32, correctly rounded.
 *
 *   k_new, v_new   [T_new, Hkv, D], f32 or bf16 (finite values)
 *   slot_mapping   i32 [T_new]; negative = row skipped; slots >= 16 * NB skipped
 *   k_cache, v_cache, k_scale, v_scale: as above, written in place
 * Supported: D in {64, 128}, page size 16.  No two rows may name the same slot.
 * T_new == 0 is a no-op.  Allocates nothing.
 */
kvs_status kv_store_paged_fp8(const kvs_tensor* k_new, const kvs_tensor* v_new,
                              const kvs_tensor* slot_mapping,
                              kvs_tensor* k_cache, kvs_tensor* v_cache,
                              kvs_tensor* k_scale, kvs_tensor* v_scale,
                              kvs_stream_t stream);

/*
 * attn_varlen_paged_fp8_ex -- attn_varlen_paged_ex over an FP8 cache (the FP8 KV
 * dispatch axis of "Transformer 추론 커널 (3/10)", §19): the same attention with K and V the dequantized values E4M3(code) * scale.
 * q, out are bf16.  `window` > 0 selects the sliding window of
 * attn_varlen_paged_window_ex (and needs causal); 0 = none.  Same paths
 * (decode and prefill / extend), shapes, limits and workspace rules as
 * attn_varlen_paged_ex.  Allocates nothing.
 */
kvs_status attn_varlen_paged_fp8_ex(const kvs_tensor* q,
                                    const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                    const kvs_tensor* k_scale, const kvs_tensor* v_scale,
                                    const kvs_tensor* block_table,
                                    const kvs_tensor* cu_seqlens_q,
                                    const kvs_tensor* seqlens_k,
                                    float scale, int causal, int32_t window,
                                    kvs_tensor* out, kvs_tensor* lse,
                                    const kvs_hints* hints,
                                    void* workspace, size_t workspace_bytes,
                                    kvs_stream_t stream);

/*
 * attn_decode_append_paged_fp8 -- the fused decode step of
 * attn_decode_append_paged over an FP8 cache ("Transformer 추론 커널 (3/10)",
 * §2 store then attention, §19 FP8 KV): sequence b's new K/V rows
 * (bf16, [B, Hkv, D]) are quantized as kv_store_paged_fp8 quantizes them
 * (codes and scales bit for bit the same) and written to the slot of key
 * Lk_b - 1, and the query row attends over the dequantized keys, the new one
 * included.  Result: kv_store_paged_fp8 then attn_varlen_paged_fp8_ex with
 * cu_seqlens_q = 0..B.  window > 0: the sliding window (0 = none).
 *
 *   k_cache, v_cache [NB, 16, Hkv, D] KVS_FP8_E4M3; k_scale, v_scale
 *   [NB, Hkv, 16] f32 (both written at the new rows); q, k_new, v_new, out bf16
 * Otherwise as attn_decode_append_paged (D = 64 or 128).  Allocates
 * nothing.
 */
kvs_status attn_decode_append_paged_fp8(const kvs_tensor* q,
                                        const kvs_tensor* k_new, const kvs_tensor* v_new,
                                        kvs_tensor* k_cache, kvs_tensor* v_cache,
                                        kvs_tensor* k_scale, kvs_tensor* v_scale,
                                        const kvs_tensor* block_table,
                                        const kvs_tensor* seqlens_k,
                                        float scale, int32_t window,
                                        kvs_tensor* out, kvs_tensor* lse,
                                        const kvs_hints* hints,
                                        void* workspace, size_t workspace_bytes,
                                        kvs_stream_t stream);

/*
 * INT8 KV cache: the same scale layout and group as the FP8 cache (one fp32
 * scale s per token row of one KV head, k_scale / v_scale [NB, Hkv, 16]);
 * codes are signed bytes c in [-127, 127] and the value of a code is c * s.
 * The pages name INT8 KV next to FP8 ("Transformer 추론 커널 (3/10)", §19,
 * §24) and fix no encoding; here the symmetric per-row form.
 *
 *   k_cache, v_cache [NB, 16, Hkv, D] dtype KVS_INT8 (codes)
 */

/*
 * kv_store_paged_int8 -- kv_store_paged_fp8 with INT8 codes ("Transformer 추론
 * 커널 (3/10)", §19: INT8 KV next to FP8): s = absmax / 127
 * (0 for an all-zero row) and code[d] = the integer nearest to x / s (ties to
 * even), clamped to +-127, both divisions in fp32, correctly rounded.  Same
 * arguments, shapes, limits and error behaviour as kv_store_paged_fp8.
 */
kvs_status kv_store_paged_int8(const kvs_tensor* k_new, const kvs_tensor* v_new,
                               const kvs_tensor* slot_mapping,
                               kvs_tensor* k_cache, kvs_tensor* v_cache,
                               kvs_tensor* k_scale, kvs_tensor* v_scale,
                               kvs_stream_t stream);

/*
 * attn_varlen_paged_int8_ex -- attn_varlen_paged_fp8_ex over an INT8 cache
 * ("Transformer 추론 커널 (3/10)", §19):
 * K and V are the dequantized values code * scale.  Same arguments, paths,
 * shapes, limits and workspace rules.  Allocates nothing.
 */
kvs_status attn_varlen_paged_int8_ex(const kvs_tensor* q,
                                     const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                     const kvs_tensor* k_scale, const kvs_tensor* v_scale,
                                     const kvs_tensor* block_table,
                                     const kvs_tensor* cu_seqlens_q,
                                     const kvs_tensor* seqlens_k,
                                     float scale, int causal, int32_t window,
                                     kvs_tensor* out, kvs_tensor* lse,
                                     const kvs_hints* hints,
                                     void* workspace, size_t workspace_bytes,
                                     kvs_stream_t stream);

/*
 * attn_decode_append_paged_int8 -- attn_decode_append_paged_fp8 over an INT8
 * cache ("Transformer 추론 커널 (3/10)", §2 and §19): the new rows are quantized as kv_store_paged_int8 quantizes them
 * (codes and scales bit for bit the same) and attended with the rest.
 * Result: kv_store_paged_int8 then attn_varlen_paged_int8_ex with
 * cu_seqlens_q = 0..B.  Same arguments and limits.  Allocates nothing.
 */
kvs_status attn_decode_append_paged_int8(const kvs_tensor* q,
                                         const kvs_tensor* k_new, const kvs_tensor* v_new,
                                         kvs_tensor* k_cache, kvs_tensor* v_cache,
                                         kvs_tensor* k_scale, kvs_tensor* v_scale,
                                         const kvs_tensor* block_table,
                                         const kvs_tensor* seqlens_k,
                                         float scale, int32_t window,
                                         kvs_tensor* out, kvs_tensor* lse,
                                         const kvs_hints* hints,
                                         void* workspace, size_t workspace_bytes,
                                         kvs_stream_t stream);

/*
 * attn_decode_append_paged_rope -- the fused decode step of
 * attn_decode_append_paged (window > 0: of attn_decode_append_paged_window)
 * with the "RoPE + KV cache store" step folded in ("Transformer 추론 커널
 * (3/10)", §2, fused with attention in one launch): q and the new key rows
 * are rotated as kv_store_rope_paged rotates them, with sequence b's new
 * token at position seqlens_k[b] - 1; the rotated key row and the unchanged
 * value row are written to the cache slot, and q is rotated in registers
 * (the q tensor is not modified).  Result: that of kv_store_rope_paged (q
 * rotated, positions Lk_b - 1, slots of key Lk_b - 1) followed by
 * attn_varlen_paged_ex / attn_varlen_paged_window_ex with cu_seqlens_q = 0..B,
 * up to rounding (the angles are reduced in double and their cos / sin taken
 * in fp32, so a rotated value may differ from kv_store_rope_paged's in its
 * last bf16 place).
 *
 * bf16 only; rotary_dim a multiple of 64 (neox) or 16 (interleaved), at most
 * D; otherwise KVS_ERR_UNSUPPORTED.  Other arguments, preconditions and limits
 * as attn_decode_append_paged.  Allocates nothing.
 */
kvs_status attn_decode_append_paged_rope(const kvs_tensor* q,
                                         const kvs_tensor* k_new, const kvs_tensor* v_new,
                                         kvs_tensor* k_cache, kvs_tensor* v_cache,
                                         const kvs_tensor* block_table,
                                         const kvs_tensor* seqlens_k,
                                         float scale, int32_t window, const kvs_rope* rope,
                                         kvs_tensor* out, kvs_tensor* lse,
                                         const kvs_hints* hints,
                                         void* workspace, size_t workspace_bytes,
                                         kvs_stream_t stream);

/* Text of the calling thread's last non-OK status ("" if none): the reason an
 * unsupported or invalid call was refused ("Transformer 추론 커널 (3/10)", §20:
 * a fallback's reason is something to record).  The pointer is valid until
 * that thread's next library call. */
const char* kvs_last_error(void);

/* Text naming the kernel variant, grid and split plan of the calling thread's
 * last successful enqueue, so a caller can log which path ran ("Transformer 추론
 * 커널 (3/10)", §20: the selected kernel's name is a metric to record). */
const char* kvs_last_dispatch(void);

/* Frees the grow-only scratch buffer (the split-KV partials of "Transformer 추론
 * 커널 (3/10)", §16) that attn_varlen_paged keeps on the current device.  A
 * teardown call: it synchronises the device first, since work queued on any
 * stream may still read the buffer.  Returns KVS_ERR_HIP if a HIP call fails. */
kvs_status kvs_release_workspace(void);


#ifdef __cplusplus
}
#endif

#endif /* KVSTORE_H */
