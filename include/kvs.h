/*
 * kvs.h -- C ABI of libkvs.so: decode attention over a head-ragged paged KV
 * cache with min-max page scoring and per-KV-head top-K page selection,
 * written for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [T] "Tangram: Unlocking Non-Uniform KV Cache Compression for Efficient
 *       Multi-turn LLM Serving" (paper review): 3.1 Budget Reservation,
 *       3.2 Ragged Paging, 3.3 AOT Load Balancing.
 *   [C] "CacheGen -- KV Cache Compression and Streaming" (paper notes):
 *       3 (change-based encoding over groups of tokens), 7 (implementation:
 *       8-bit anchors, a delta bin per third of the layers, arithmetic
 *       coding with statistics per channel and layer, GPU decoding).
 *   [F] "FlexiCache: Leveraging Temporal Stability of Attention Heads for
 *       Efficient KV Cache Management (MLSys 2026)" (paper summary): Core
 *       method (sparse decode, Quest-style min-max page bound), Method
 *       (stable and unstable heads, rerank every 16 steps for stable heads,
 *       no scoring between reranks), System engineering (per-head-layer
 *       block table with null blocks; physical block reuse in the
 *       rerank kernel; transfer kernel over pinned host memory), Key
 *       observations, assumption 2 (GPU-resident MinMax cache), tiered
 *       placement (stable heads keep their top-K pages on the GPU, the
 *       rest in host memory; only newly promoted pages move).
 *
 * Conventions shared by every call
 *   - Return value: KVS_OK (0) or a negative KVS_E* code.  On error no kernel
 *     was launched and kvs_last_error() (thread-local) holds a message.  A
 *     failed launch returns KVS_EHIP with the HIP error text.
 *   - Device calls are asynchronous and ordered on `stream` (a hipStream_t
 *     passed as void*; NULL = the default stream).  Host-only calls are
 *     synchronous and touch no device.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device memory and keeps no pointer after a call returns; scratch space
 *     comes from the caller's `workspace`.  Calls are reentrant.
 *   - Layout is row-major C order throughout.  Element types: KV, min-max
 *     and queries are fp16 or bf16 (`dtype`), scores and outputs fp32,
 *     indices int32.  Device pointers must be 16-byte aligned.
 *   - Contents of device-resident integer inputs (seq_len, page_table,
 *     meta_base, sel) cannot be checked before launch.  Kernels never read
 *     outside the buffers described here: a page id outside [0, num_pages)
 *     or a negative id is treated as a null page and skipped (only scoring
 *     and the host tier calls tell KVS_PAGE_ON_HOST apart), as is a
 *     min-max block outside [0, num_meta); seq_len is clamped to
 *     [0, P*max_group_pages]; sel_count is clamped to [0, K].
 */
#ifndef KVS_H_
#define KVS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVS_OK = 0,
  KVS_EINVAL = -1,        /* bad argument (null, misaligned, out of range) */
  KVS_EUNSUPPORTED = -2,  /* valid but not built: head_dim, page size, dtype, GQA */
  KVS_EHIP = -3,          /* HIP runtime error */
  KVS_ENOSPC = -4         /* caller's workspace too small */
};

enum { KVS_F16 = 0, KVS_BF16 = 1 };

/* Page-table entry of a logical page whose K/V lives only in the host tier
 * (kvs_host_tier): its bounds are on the GPU, so it is scored like a
 * resident page, but the decode skips it until kvs_promote_pages maps it. */
#define KVS_PAGE_ON_HOST (-2)

/*
 * One layer's head-ragged paged KV cache [T 3.2; F System engineering].
 *
 * KV heads are cut into G = Hkv/Hp groups of Hp heads; each group has its
 * own page table.  A physical page holds, for each of the group's Hp heads,
 * P tokens of K followed by P tokens of V:
 *     kv[num_pages][Hp][2][P][d]         (index 2: 0 = K, 1 = V)
 * so one head's K tile of a page is P*d contiguous elements.
 * A group is allocated pages for its longest head [T 3.2]; shorter heads of
 * the group leave the tail of their slots unused.
 *
 *   kv          device, [num_pages][Hp][2][P][d] dtype.  Written by the
 *               appends and kvs_promote_pages.
 *   minmax      device, [num_meta][d][2] dtype: the min-max cache [F Key
 *               observations, assumption 2], kept apart from the KV pages
 *               and ragged per head: block meta_base[r][h] + p holds, for
 *               logical page p of head h of request r, per channel the
 *               minimum (index 0) then the maximum (index 1) of the valid
 *               keys.  A head's bounds are one contiguous run in page order
 *               however its KV pages are scattered.  Written by
 *               kvs_build_minmax, read by kvs_score_pages.
 *   meta_base   device, [b][Hkv] int32: first minmax block of each head; the
 *               head's run holds ceil(n/P) blocks.
 *   page_table  device, [b][G][max_group_pages] int32 physical page ids;
 *               -1 marks a null entry [F System engineering],
 *               KVS_PAGE_ON_HOST a page held in the host tier.  Logical
 *               page p of head h covers its tokens [p*P, (p+1)*P).  Written
 *               only by kvs_promote_pages (tiered heads' entries).
 *   seq_len     device, [b][Hkv] int32: n, the tokens head h of request r
 *               holds (ceil(B*N) retained under Budget Reservation [T 3.1],
 *               plus the tokens appended since), 0 <= n <= P*max_group_pages
 *               (n = 0: a head with no token yet, e.g. before the first
 *               prefill chunk).
 *               Written only by the appends (kvs_append_kv,
 *               kvs_append_kv_tier) and kvs_prefill_chunk.
 *   head_slot   device, [Hkv] int32: head h sits in group head_slot[h]/Hp,
 *               slot head_slot[h]%Hp; a permutation of [0, Hkv).
 *   b, Hq, Hkv  requests, query heads, KV heads (Hq % Hkv == 0).
 *   Hp          heads per page group (Hkv % Hp == 0, G <= 64).
 *   num_meta    blocks in minmax.
 *   d           head dimension: 128 or 256.
 *   P           tokens per page: 16.
 *   dtype       KVS_F16 or KVS_BF16.
 */
typedef struct kvs_paged_kv {
  void* kv;
  void* minmax;
  const int32_t* meta_base;
  const int32_t* page_table;
  int32_t* seq_len;
  const int32_t* head_slot;
  int32_t b, Hq, Hkv, Hp, d, P, max_group_pages, num_pages, num_meta, dtype;
} kvs_paged_kv;

/*
 * Build the min-max page metadata [F Key observations, assumption 2; Core
 * method].  For every request r, head h and logical page p < ceil(n/P):
 * minmax[meta_base[r][h] + p][c][0] = min and [c][1] = max over the page's
 * valid tokens t in [p*P, min(n, (p+1)*P)) of K[t][c].  Exact (a
 * selection).  Pages with a null table entry and block indices outside
 * [0, num_meta) are skipped.
 * Blocks of pages beyond a head's n are left untouched.
 * Runs once per page fill, not per decode step.  Needs b*Hkv <= 16383
 * (KVS_EUNSUPPORTED otherwise).
 */
int kvs_build_minmax(const kvs_paged_kv* cache, void* stream);

/*
 * Quest-style page scores [F Core method].  For request r, KV head h and
 * logical page p < ceil(n/P):
 *   scores[r][h][p] = max over the Gq query heads g of h of
 *                     sum_c max(q[r][g][c]*kmin[c], q[r][g][c]*kmax[c])
 * (no 1/sqrt(d) scale), fp32 products of the fp16/bf16 inputs (exact) summed
 * in a fixed order.  Pages p >= ceil(n/P), pages with a null table entry and
 * pages whose block is outside [0, num_meta) get -inf; a KVS_PAGE_ON_HOST
 * page is scored from its bounds like a resident one.
 *   q       device, [b][Hq][d] dtype; query head g belongs to KV head g/Gq.
 *   scores  device, [b][Hkv][max_group_pages] fp32, fully written.
 * Supported sizes: b*Hkv <= 16383 and b*Hkv*max_group_pages < 2^31
 * (KVS_EUNSUPPORTED otherwise).
 */
int kvs_score_pages(const kvs_paged_kv* cache, const void* q, float* scores, void* stream);

/*
 * kvs_score_pages restricted to the KV heads h with heads[h] != 0 (host
 * array [Hkv], the same for every request): stable heads are not scored
 * between their reranks, and a layer whose heads are all stable is not
 * scored at all [F Method].  Score rows of the other heads are left
 * untouched.  The heads array is read before the call returns.
 */
int kvs_score_pages_heads(const kvs_paged_kv* cache, const void* q, const uint8_t* heads,
                          float* scores, void* stream);

/*
 * Per-KV-head top-K page selection [F Core method].  For each (r, h) with
 * np = ceil(seq_len[r][h]/P) pages: keep the min(K, np) pages of largest
 * score, equal scores going to the lower page index, and write them in
 * ascending page order.  Integer keys built from the fp32 bits (value
 * order; -0 and +0 are equal).  Deterministic.
 *   scores     device, [b][Hkv][max_pages] fp32 (entries >= np ignored).
 *   seq_len    device, [b][Hkv] int32.
 *   K          1 <= K <= 1024.  max_pages <= 8192.
 *   sel        device, [b][Hkv][K] int32; entries >= sel_count are -1.
 *   sel_count  device, [b][Hkv] int32 = min(K, np).
 */
int kvs_topk_pages(const float* scores, const int32_t* seq_len, int32_t P, int32_t b,
                   int32_t Hkv, int32_t max_pages, int32_t K, int32_t* sel,
                   int32_t* sel_count, void* stream);

/*
 * kvs_topk_pages restricted to the KV heads h with heads[h] != 0 (host array
 * [Hkv]); the other heads keep the selection they hold, sel and sel_count
 * untouched -- a stable head reuses the pages of its last rerank [F Method].
 */
int kvs_topk_pages_heads(const float* scores, const int32_t* seq_len, int32_t P, int32_t b,
                         int32_t Hkv, int32_t max_pages, int32_t K, const uint8_t* heads,
                         int32_t* sel, int32_t* sel_count, void* stream);

/*
 * kvs_score_pages followed by kvs_topk_pages with K, in one launch [F Core
 * method]: the same scores, bit for bit, and the same selection.  One
 * workgroup per (request, KV head) scores the head's pages into on-chip
 * memory and selects from there, so a head's scores are never re-read and
 * the selection needs no launch of its own; it pays off when the b*Hkv heads
 * are many and of similar length (a long head holds its workgroup while the
 * others idle).
 *   q          as kvs_score_pages.
 *   scores     device, [b][Hkv][max_group_pages] fp32 written as
 *              kvs_score_pages writes it, or NULL: the scores are not stored.
 *   K          1 <= K <= 1024.  max_group_pages <= 8192.
 *   sel, sel_count  as kvs_topk_pages.
 * Errors: the descriptor, q, K and max_group_pages checks of the two calls
 * it replaces (KVS_EINVAL, KVS_EUNSUPPORTED), except the scoring's b*Hkv
 * limit, which does not apply (one workgroup per head, no page-count scan);
 * a launch failure gives KVS_EHIP.  Nothing is launched on an error.
 */
int kvs_select_pages(const kvs_paged_kv* cache, const void* q, float* scores, int32_t K,
                     int32_t* sel, int32_t* sel_count, void* stream);

/*
 * Append the decoded token of every head to its ragged page [F Method: the
 * token being decoded joins the cache; T 3.2 Ragged Paging] and update that
 * page's min-max bounds in place [F Key observations, assumption 2].  For
 * every (r, h) with n = seq_len[r][h] < P*max_group_pages: K and V of the
 * token go to row n % P of logical page p = n / P in the head's slot;
 * block meta_base[r][h] + p becomes (k, k) per channel if the row is the
 * page's first, else (min(kmin, k), max(kmax, k)) (exact: a selection);
 * then seq_len[r][h] = n + 1.
 *   k_new, v_new  device, [b][Hkv][d] dtype, 16-byte aligned.
 * The caller maps page p in the page table and owns block meta_base[r][h] +
 * p before the call.  A head whose page entry is null or outside the pool,
 * whose block lies outside [0, num_meta), or whose n is already
 * P*max_group_pages is left as it is (token, bounds and n unchanged).
 */
int kvs_append_kv(const kvs_paged_kv* cache, const void* k_new, const void* v_new, void* stream);

/*
 * One chunk of a chunked prefill under Budget Reservation [T 3.1: as each
 * chunk's K/V is computed, every head keeps its top tokens by a score, so the
 * compressed footprint is fixed at scheduling and nothing is reclaimed]:
 * for every (r, h) with n = seq_len[r][h], keep the q = quota[r][h] tokens
 * of the chunk with the largest score (equal scores to the lower position),
 * write them in position order to positions n .. n+q-1 of the head's slot
 * in its group's pages [T 3.2], update the min-max bounds of every page they
 * land in [F Key observations, assumption 2] (merged with the bounds the
 * first page already held), and set seq_len[r][h] = n + q.  q is clamped to
 * [0, min(C, P*max_group_pages - n)].  The quota is an input; the reading
 * used here, chunk [a, e) of an N-token prompt keeps ceil(B e) - ceil(B a)
 * tokens (ceil(B N) in all), is what kvs_prefill_quota computes.
 *   k_chunk, v_chunk  device, [b][Hkv][C][d] dtype, 16-byte aligned.
 *   scores            device, [b][Hkv][C] fp32 (integer keys from the fp32
 *                     bits, as in kvs_topk_pages).
 *   quota             device, [b][Hkv] int32.
 *   C                 chunk length, 1 <= C <= 8192.  Positions past a
 *                     request's prompt must carry -inf scores; the quota
 *                     never exceeds the number of the others.
 *   workspace         device scratch of at least
 *                     kvs_prefill_workspace_bytes(b, Hkv, C) bytes, 256-byte
 *                     aligned; contents on entry do not matter.
 *   b*Hkv <= 65535 (KVS_EUNSUPPORTED otherwise).
 * The pages for positions n .. n+q-1 must be mapped and the head must own
 * blocks meta_base[r][h] + p for them (the reservation).  A token whose page
 * entry is null is not written; a head whose head_slot is out of range is
 * left as it is.
 */
int kvs_prefill_chunk(const kvs_paged_kv* cache, const void* k_chunk, const void* v_chunk,
                      const float* scores, const int32_t* quota, int32_t C, void* workspace,
                      size_t ws_bytes, void* stream);

/* Bytes of workspace kvs_prefill_chunk needs (per head: its length before
 * the chunk, its quota and the kept positions).  0 on bad arguments. */
size_t kvs_prefill_workspace_bytes(int32_t b, int32_t Hkv, int32_t C);

/*
 * Budget Reservation quota of one prefill chunk, host only [T 3.1: every
 * head keeps Top(ceil(B N), s) of its N-token prompt, chunk by chunk, so its
 * footprint is fixed when the request is scheduled].  Reading: after the
 * first x tokens a head has kept ceil(B x) (0 for x = 0), so the chunk of
 * positions [start, start + chunk) keeps, for request r and head h,
 *   quota[r][h] = ceil(B_h e) - ceil(B_h a),
 *   a = min(N_r, start), e = min(N_r, start + chunk),
 * which telescopes to ceil(B_h N_r) over all chunks and never exceeds the
 * chunk's length.  The ceiling is taken on the exact binary value of B_h
 * (integer arithmetic, no rounding).
 *   budgets   host, [Hkv] double in (0, 1]: one layer's head budgets.
 *   contexts  host, [b] int64 in [1, 2^40]: prompt length per request.
 *   start     first position of the chunk, 0 <= start <= 2^40; chunk >= 1.
 *   quota     host out, [b][Hkv] int32 (the input of kvs_prefill_chunk,
 *             once copied to the device).
 * KVS_EINVAL on a null pointer or any value out of range, before any write.
 */
int kvs_prefill_quota(const double* budgets, const int64_t* contexts, int32_t b, int32_t Hkv,
                      int64_t start, int32_t chunk, int32_t* quota);

/*
 * Heads that re-select their pages at a decode step, host only [F Method:
 * heads whose attention is stable over steps reuse their page selection
 * between periodic reranks; the others re-select every step].  Reading:
 * steps count from the first decode step (step 0), which always selects, so
 *   due[h] = (step % period == 0) || !stable[h].
 *   stable   host, [Hkv] bytes, nonzero = stable head.
 *   due      host out, [Hkv] bytes, 1 = re-select (the head mask of
 *            kvs_score_pages_heads / kvs_topk_pages_heads).
 * KVS_EINVAL on a null pointer, Hkv < 1, step < 0 or period < 1.
 */
int kvs_rerank_heads(const uint8_t* stable, int32_t Hkv, int32_t step, int32_t period,
                     uint8_t* due);

/*
 * Host tier of a cache whose stable heads keep only their selected pages on
 * the GPU [F tiered placement].  Needs Hp == 1, so that every head has a
 * page table of its own.  A tiered head (host_base[r][h] >= 0) has every
 * logical page p < ceil(n/P) in host memory at host page host_base[r][h] + p
 * and owns `slots` GPU pages; its table entry for p is the physical id of
 * the slot holding p when p is resident and KVS_PAGE_ON_HOST otherwise.
 * Heads with host_base < 0 are not tiered and keep all pages on the GPU.
 *   host_kv         pinned host memory allocated by hipHostMalloc (torch's
 *                   pin_memory allocator is one), [num_host_pages][2][P][d]
 *                   dtype: the same K-then-V tile as a GPU page.  Kernels
 *                   read and write it directly over the host link; the
 *                   call checks that the pointer is pinned host memory
 *                   mapped for the device and fails with KVS_EINVAL if not.
 *                   It cannot check the size: the caller guarantees
 *                   num_host_pages pages.
 *   host_base       device, [b][Hkv] int64.
 *   slot_page       device, [b][Hkv][slots] int32: the logical page held by
 *                   each GPU slot of the head, -1 when free.  Written only by
 *                   kvs_promote_pages.
 *   slot_phys       device, [b][Hkv][slots] int32: the physical page of each
 *                   slot (ids outside [0, num_pages) mark unusable slots).
 *   slots           GPU pages per tiered head, 1 <= slots <= 1024.
 *   num_host_pages  pages in host_kv, 1 <= num_host_pages < 2^31.
 */
typedef struct kvs_host_tier {
  void* host_kv;
  const int64_t* host_base;
  int32_t* slot_page;
  const int32_t* slot_phys;
  int32_t slots;
  int64_t num_host_pages;
} kvs_host_tier;

/*
 * Bulk offload after prefill [F tiered placement]: for every tiered head,
 * every page p < ceil(n/P) whose table entry is a physical page is copied
 * from the GPU to host page host_base[r][h] + p.  Reads only host_kv,
 * host_base and num_host_pages of the tier; the table is not changed (the
 * caller remaps the head once the copy has completed on `stream`).  Host
 * pages outside [0, num_host_pages) are skipped.  Needs b*Hkv <= 65535.
 */
int kvs_offload_pages(const kvs_paged_kv* cache, const kvs_host_tier* tier, void* stream);

/*
 * kvs_append_kv on a cache with a host tier [F tiered placement: a stable
 * head's pages, newly filled ones included, live in host memory].  For a
 * tiered head the K and V rows are written through to host page
 * host_base[r][h] + n/P (row n%P), and also to the GPU page when the table
 * maps that page; its bounds are merged and n advances as in kvs_append_kv.
 * The host copy of every page thus stays complete, and a later promotion
 * brings the new rows along.  A tiered head whose host page is outside
 * [0, num_host_pages) is skipped (n unchanged).  Other heads: kvs_append_kv.
 * Reads only host_kv, host_base and num_host_pages of the tier.
 */
int kvs_append_kv_tier(const kvs_paged_kv* cache, const kvs_host_tier* tier, const void* k_new,
                       const void* v_new, void* stream);

/*
 * Promotion after a rerank [F tiered placement; physical block reuse in the
 * rerank kernel; transfer kernel over pinned host memory].  For every tiered
 * head h with heads[h] != 0 (heads: host array [Hkv], NULL = every head)
 * and the selection sel[r][h][0 .. sel_count) of kvs_topk_pages:
 *   - a slot whose page is not selected is freed; that page's entry becomes
 *     KVS_PAGE_ON_HOST (p < ceil(n/P)) or -1 (beyond);
 *   - a selected page p < ceil(n/P) whose entry is KVS_PAGE_ON_HOST is
 *     promoted: copied from host page host_base[r][h] + p into a free slot
 *     (free slots in slot order, promoted pages in ascending page order),
 *     whose physical id becomes the entry; pages already resident stay
 *     where they are, so only the set difference crosses the host link.
 * Afterwards every selected page of the head is resident and no other page
 * is, provided slots >= K.  Heads not tiered or not in `heads` are left as
 * they are.
 *   sel, sel_count  device, as written by kvs_topk_pages with this K.
 *   K               1 <= K <= slots.
 *   moved           device, [b][Hkv] int32 or NULL: pages copied per head
 *                   (0 for heads left as they are).
 * Needs max_group_pages <= 8192 and b*Hkv <= 2^31 - 1.  Calls overlapping
 * on one cache race; the decode after it must be ordered after it.
 */
int kvs_promote_pages(const kvs_paged_kv* cache, const kvs_host_tier* tier, const int32_t* sel,
                      const int32_t* sel_count, int32_t K, const uint8_t* heads, int32_t* moved,
                      void* stream);

/*
 * Ahead-of-time workload split map [T 3.3], host only.
 * Per layer l: weight w_h = round(min(B[l][h], cap) * 2^20) (cap <= 0: no
 * cap), group load phi_i = sum of w_h over the heads with head_slot/Hp == i,
 * then T splits are apportioned by highest averages (D'Hondt): every group
 * starts with 1, each further split goes to the largest phi_i/S_i (exact
 * integer comparison, equal loads to the lower i).  This minimises the
 * largest load per split; the page states only that goal and the
 * proportionality, not the algorithm.
 *   budgets    host, [L][Hkv] in (0, 1].
 *   head_slot  host, [L][Hkv], each row a permutation of [0, Hkv).
 *   T          splits per request per layer, G <= T <= 65536.
 *   S          host out, [L][G] int32, each row sums to T.
 */
int kvs_plan_split(const double* budgets, const int32_t* head_slot, int32_t L, int32_t Hkv,
                   int32_t Hp, double cap, int32_t T, int32_t* S);

/*
 * Ragged split-K decode attention plus LSE combine [F Core method; T 3.2,
 * 3.3].  For request r and group i the work units are the group's (slot,
 * page) pairs, head-major: slot 0's attended pages in list order, then slot
 * 1's, ...  A head attends its sel list (sel_count entries) when sel is
 * non-NULL, else all of its ceil(n/P) pages.  With U units and S_i =
 * S_row[i] splits, split s takes units [floor(s*U/S_i), floor((s+1)*U/S_i)).
 * One workgroup per (r, i, s) computes, for every query head of every head
 * it touches, softmax(scale * q.k) v over the valid tokens of its units and
 * the log-sum-exp; a second kernel merges the splits of each query head:
 *   out[r][g] = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, M = max lse_s.
 *   q          device, [b][Hq][d] dtype.
 *   sel        device, [b][Hkv][K] int32 or NULL; sel_count device [b][Hkv].
 *   K          row length of sel (ignored when sel is NULL).
 *   S_row      host, [G] int32, each >= 1, sum <= 65536; b*sum(S_row)
 *              workgroups are launched.
 *   scale      softmax scale, usually 1/sqrt(d).
 *   workspace  device scratch of at least kvs_decode_workspace_bytes(...)
 *              bytes, 256-byte aligned; contents on entry do not matter.
 *   out        device, [b][Hq][d] fp32.  A query head whose KV head has no
 *              valid token in its attended pages (n = 0, an empty
 *              selection, or only null pages) gets a zero row: attention
 *              over no token is taken as the empty sum.
 */
int kvs_decode_attn(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                    const int32_t* sel_count, int32_t K, const int32_t* S_row, float scale,
                    void* workspace, size_t ws_bytes, float* out, void* stream);

/*
 * The two phases of kvs_decode_attn as calls of their own: the ragged
 * split-K decode [T 3.2, 3.3] and the log-sum-exp combine of the splits [F
 * Core method].  Both take exactly kvs_decode_attn's arguments and make its
 * checks; kvs_decode_splits launches only the split kernel, which writes
 * every split's partial output and log-sum-exp (and each head's first and
 * last split) into `workspace`; kvs_decode_combine launches only the
 * combine, which reads them from `workspace` and writes `out`.  The two
 * called in that order on one stream, with the same arguments and workspace
 * (and nothing writing that workspace in between), give bit for bit the
 * output of one kvs_decode_attn call.  kvs_decode_combine on a workspace no
 * kvs_decode_splits call has filled for these arguments reads whatever the
 * workspace holds (finite or not): the result is then undefined, though
 * every access stays inside the workspace and `out`.  q and scale are
 * checked but not used by kvs_decode_combine; out is not written by
 * kvs_decode_splits.
 */
int kvs_decode_splits(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                      const int32_t* sel_count, int32_t K, const int32_t* S_row, float scale,
                      void* workspace, size_t ws_bytes, float* out, void* stream);
int kvs_decode_combine(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                       const int32_t* sel_count, int32_t K, const int32_t* S_row, float scale,
                       void* workspace, size_t ws_bytes, float* out, void* stream);

/*
 * kvs_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from scratch memory
 * the library holds instead of a caller argument.  Allocates nothing: no
 * hipMalloc, hipFree or allocating library call.  The caller still passes
 * the inputs and `out` as for kvs_decode_attn.
 *   Scratch: one array of KVS_NOALLOC_SCRATCH_BYTES (64 MiB) per device,
 *   a file-scope device array of the library, present from the library's
 *   load until the process ends.  Its device address is looked up on the
 *   first call on each device (the only HIP call besides the launches).
 *   A shape and split row whose kvs_decode_workspace_bytes exceeds it is
 *   rejected with KVS_ENOSPC before anything runs (e.g. 64 requests x 16
 *   query heads x head_dim 256 allow up to 63 splits per group).
 *   Every call on a device shares that device's array and leaves its last
 *   contents there (nothing in it needs to start at any value): calls that
 *   overlap on one device -- on different streams or host threads -- race
 *   and must be ordered by the caller.
 */
#define KVS_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int kvs_decode_attn_noalloc(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                            const int32_t* sel_count, int32_t K, const int32_t* S_row,
                            float scale, float* out, void* stream);

/* Bytes of workspace kvs_decode_attn needs for this shape and split row
 * (per-split partial outputs and log-sum-exps, and each head's first and
 * last split).  0 on bad arguments. */
size_t kvs_decode_workspace_bytes(int32_t b, int32_t Hq, int32_t Hkv, int32_t d,
                                  const int32_t* S_row, int32_t G);

/* Concurrent decode workgroups on `device` for this kernel variant [T 3.3:
 * the split map is sized to what the chip runs at once]:
 * *W = compute units x max resident workgroups per compute unit. */
int kvs_decode_concurrency(int32_t device, int32_t d, int32_t gqa, int32_t dtype, int32_t* W);

/*
 * Read probe of the decode's gather, a measurement aid (the empirical HBM
 * ceiling of the decode's access pattern): for every (r, h) and each unit
 * the decode attends -- sel[r][h][0 .. sel_count) clamped to the head's
 * pages as in kvs_decode_attn, or every page when sel is NULL -- it reads
 * that page's whole K and V tile of head h through the page table, with no
 * arithmetic.  The XOR of all 32-bit words read by a wave is written to one
 * sink word per wave; sink words past the grid's waves are untouched.  A
 * null page counts for nothing (its loads go to page 0 and are not folded).
 * The XOR over the sink words therefore equals the XOR of every word of the
 * attended tiles of mapped pages.
 *   sink        device, sink_words >= kvs_gather_probe_sink_words(d)
 *               (KVS_ENOSPC otherwise).
 * Needs b*Hkv <= 16383.
 */
int kvs_gather_probe(const kvs_paged_kv* cache, const int32_t* sel, const int32_t* sel_count,
                     int32_t K, uint32_t* sink, size_t sink_words, void* stream);

/* Sink words kvs_gather_probe needs on the current device for head_dim d. */
int kvs_gather_probe_sink_words(int32_t d, int32_t* words);

/*
 * Plain read probe, a measurement aid (the chip's read rate for one launch
 * of a given size, with no gather): reads the `bytes` contiguous bytes at
 * src with the non-temporal 16-byte loads the kernels use, each wave of a
 * resident grid an even contiguous share, and writes the XOR of the 32-bit
 * words each wave read to one sink word per wave (sink words past the grid's
 * waves are untouched); the XOR over the sink words is the XOR of every word
 * read.
 *   src         device, 16-byte aligned; bytes a positive multiple of 16
 *               (KVS_EINVAL otherwise).
 *   sink        device, sink_words >= kvs_stream_probe_sink_words (KVS_ENOSPC
 *               otherwise).
 */
int kvs_stream_probe(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                     void* stream);

/* Sink words kvs_stream_probe needs on the current device. */
int kvs_stream_probe_sink_words(int32_t* words);

/*
 * KV-cache codec [C 3, 7]: one chunk of T tokens of every layer,
 *     x[L][2][T][C] fp16 (index 1: 0 = K, 1 = V; C = all KV heads' channels
 *     of a token side by side),
 * coded as follows.
 *   - Token t is the anchor of its group iff t % group == 0.  An anchor is
 *     kept at 8 bits: code = round((x - lo) / scale) in [0, 255], with lo and
 *     hi the min and max of the chunk's anchors of that (layer, K/V,
 *     channel) and scale = (hi - lo) / 255 (0 for a constant channel: code
 *     0).  Any other token stores q = round((x - x_anchor) / bin) clamped to
 *     [-127, 127] against its group's original anchor value, with
 *     bin = bins[floor(3 l / L)] for layer l.  Rounding is half to even,
 *     all in IEEE float32.
 *   - Decoded values: an anchor is lo + code*scale; another token is its
 *     anchor's decoded value + q*bin; float32, product then sum, rounded once
 *     to fp16.
 *   - Every (layer, K/V, channel) has two frequency tables, kind 0 for
 *     anchors and 1 for deltas, built from the chunk's own symbols: over the
 *     symbols first .. first + n - 1 (the smallest to the largest present),
 *     floor(count * 2^16 / total), at least 1 for a present symbol, 0 for an
 *     absent one; the rounding difference goes to the largest frequency
 *     (ties: the lowest symbol).  A kind with no symbols has the single
 *     symbol 0 at 2^16.
 *   - A stream holds one token's symbols over S consecutive channels, in
 *     channel order, range coded (32-bit, byte-wise, carry propagating:
 *     r = floor(range / 2^16), renormalised while range < 2^24, five
 *     flushing shifts), padded with zero bytes to a multiple of 4.  Streams
 *     are stored in order ((l*2 + kv)*(C/S) + slice)*T + t.
 */
typedef struct kvs_codec_layout {
  int32_t L, T, C;   /* layers, tokens, channels per token */
  int32_t group;     /* tokens per group, 1 .. 320 (10 in [C 3]) */
  int32_t S;         /* channels per stream: a multiple of 8 dividing C */
  float bins[3];     /* delta bins of the layer thirds, > 0 ([C 7]: 0.5, 1, 1.5) */
} kvs_codec_layout;

/*
 * An encoded chunk.  Table i = ((l*2 + kv)*C + c)*2 + kind.
 *   lo, scale      [L][2][C] float32: the anchors' code range.
 *   tab_first      [L][2][C][2] int32: first symbol of table i.
 *   tab_n          [L][2][C][2] int32: symbols in table i (1 .. 256).
 *   tab_off        [L][2][C][2] uint32: table i's cumulative frequencies
 *                  start at cdf[tab_off[i]]; tables are stored in index
 *                  order, back to back.
 *   cdf            uint16: entry j of table i is the sum of the frequencies
 *                  of its symbols before j (entry 0 is 0; the total 2^16
 *                  after the last entry is implied).
 *   cdf_len        entries of cdf (capacity on input to kvs_codec_encode,
 *                  entries written on return).
 *   streams        the streams' bytes; stream k is streams[stream_off[k] ..
 *                  stream_off[k+1]).
 *   stream_off     [L*2*(C/S)*T + 1] uint64 byte offsets (multiples of 4).
 *   streams_len    bytes of streams (capacity on input to kvs_codec_encode,
 *                  bytes written on return).
 */
typedef struct kvs_codec_chunk {
  float* lo;
  float* scale;
  int32_t* tab_first;
  int32_t* tab_n;
  uint32_t* tab_off;
  uint16_t* cdf;
  uint64_t cdf_len;
  uint8_t* streams;
  uint64_t* stream_off;
  uint64_t streams_len;
} kvs_codec_chunk;

/* Upper bounds of cdf_len and streams_len for a layout (host only; 0 for an
 * invalid layout). */
int kvs_codec_bounds(const kvs_codec_layout* layout, uint64_t* cdf_max, uint64_t* streams_max);

/*
 * Encode one chunk on the host (offline, as in [C 3]): x is host memory,
 * every buffer of `out` host memory sized per `layout` (lo, scale:
 * L*2*C; tab_*: L*2*C*2; stream_off: L*2*(C/S)*T + 1).  Runs on up to
 * `threads` host threads (0: the hardware's count).  KVS_ENOSPC when
 * cdf_len or streams_len is too small, with the sizes needed written to
 * them; nothing else is then guaranteed written.
 */
int kvs_codec_encode(const kvs_codec_layout* layout, const uint16_t* x, kvs_codec_chunk* out,
                     int32_t threads);

/*
 * Decode one chunk on the GPU [C 7]: every buffer of `chunk` is device
 * memory holding what kvs_codec_encode wrote; out is device
 * [L][2][T][C] fp16, fully written (streams_len >= 8: every stream has at
 * least 8 bytes).  One lane decodes one stream; the
 * kernel never reads outside the buffers described by cdf_len and
 * streams_len (a corrupt stream decodes to garbage, not a fault).
 * Needs C/S*L*2 <= 65535 workgroup rows and T <= 2^31 / 2.
 */
int kvs_codec_decode(const kvs_codec_layout* layout, const kvs_codec_chunk* chunk, void* out,
                     void* stream);

/* Budget-aware clustering [T 3.2], host only: per layer, heads ordered by
 * budget (largest first, equal budgets by lower head index); the head at
 * sorted position pos gets head_slot = pos (group pos/Hp, slot pos%Hp).
 *   budgets [L][Hkv] host; head_slot [L][Hkv] host out. */
int kvs_cluster_heads(const double* budgets, int32_t L, int32_t Hkv, int32_t Hp,
                      int32_t* head_slot);

/* Message of the last error on this thread ("" if none). */
const char* kvs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H_ */
