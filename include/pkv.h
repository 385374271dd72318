/*
 * pkv.h -- C ABI of libpkv, the paged KV-cache decode path for AMD Instinct MI355X (gfx950).
 *
 * The method ("PagedAttention: Efficient LLM Serving with vLLM", "How PagedAttention Works";
 * "Efficient Memory Management for Large Language Model Serving with PagedAttention",
 * Abstract and observer card "Key ideas"): each sequence's key/value cache is cut into
 * fixed-size blocks of block_size tokens (16 by default) that sit anywhere in a physical
 * block pool; a per-sequence block table maps logical block j to its physical block; decode
 * attention gathers K/V through that table; new tokens are written into the slot the block
 * manager hands out; sequences that share a prefix share its blocks until one of them writes
 * (copy-on-write).
 *
 * Conventions for every call below
 *   - Device pointers are plain addresses in the current HIP device's memory; host pointers
 *     are marked "host".  The caller owns every device buffer (the library never allocates
 *     or frees device memory).  Only the block manager and the step driver keep pointers
 *     beyond a call, as stated there.
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *     null stream) and never synchronize.  Argument errors are detected on the host before
 *     anything is launched and returned as a status; nothing is launched then.
 *   - Pool layout (K and V alike): [num_blocks][num_heads][block_size][head_dim], element type
 *     `dtype`, row-major, contiguous.  Token t of a sequence lives in physical block
 *     block_table[t / block_size] at slot t % block_size.  A "slot" number is
 *     physical_block * block_size + offset.
 *   - Supported shapes: head_dim in {64, 128}; block_size in {8, 16, 32}; dtype f32, f16, bf16;
 *     otherwise PKV_EUNSUPPORTED.
 *   - Device index arrays (block tables, context lengths, slot mappings, copy pairs) are read
 *     by the kernels and cannot be checked on the host.  Out-of-range entries never cause an
 *     out-of-bounds access: see each call for what they produce instead.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* a null pointer, a negative or inconsistent size, an unknown id */
  PKV_EUNSUPPORTED = 2,  /* a shape or dtype the library has no kernel for */
  PKV_ENOMEM = 3,        /* block pool exhausted (allocator) or workspace too small */
  PKV_EHIP = 4           /* the HIP runtime reported an error at launch */
} pkv_status_t;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype_t;

/* Shape of one layer's K (or V) block pool. */
typedef struct {
  int32_t num_blocks;  /* physical blocks in the pool */
  int32_t num_heads;   /* KV heads (one query head per KV head) */
  int32_t block_size;  /* tokens per block: 8, 16 or 32 */
  int32_t head_dim;    /* 64 or 128 */
  int32_t dtype;       /* pkv_dtype_t of the pool, of q / out and of new k / v */
} pkv_cache_desc_t;

typedef void* pkv_stream_t; /* a hipStream_t */

int32_t pkv_abi_version(void);
const char* pkv_status_string(pkv_status_t status);

/* ---------------------------------------------------------------------------------------
 * Paged decode attention.
 * ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
 * steps 4-5: the page table maps logical to physical blocks and attention gathers the
 * scattered K/V pairs through it.)
 *
 * For every sequence s < num_seqs and head h < num_heads, with L = context_lens[s]:
 *     z_t = scale * <q[s][h][:], K(s, t, h)>      for t = 0 .. L-1
 *     out[s][h][:] = sum_t softmax(z)_t * V(s, t, h)
 * where K(s, t, h) = k_pool[block_tables[s * max_blocks_per_seq + t / block_size]][h]
 *                          [t % block_size][:], and V alike.  Arithmetic is binary32 with
 * binary32 accumulation; out is rounded to dtype (round to nearest even).  L = 0 gives a zero
 * vector.  The new token is attended like any other: append it first (pkv_reshape_and_cache),
 * then pass its length including it.
 *
 *   out           device, [num_seqs][num_heads][head_dim], dtype; written
 *   q             device, [num_seqs][num_heads][head_dim], dtype
 *   k_pool,v_pool device, pool layout above
 *   block_tables  device, int32 [num_seqs][max_blocks_per_seq]; entries past a sequence's
 *                 last block are never read
 *   context_lens  device, int32 [num_seqs]; a value above max_context_len or above
 *                 max_blocks_per_seq * block_size is clamped to the smaller of the two, a
 *                 negative value reads as 0
 *   max_context_len  host; an upper bound of context_lens, sizes the launch and workspace
 *   scale         host; the softmax temperature (usually 1/sqrt(head_dim))
 *   workspace     device, >= pkv_decode_workspace_bytes(...) bytes, 16-byte aligned; may be
 *                 NULL when that size is 0.  Scratch for the split-context partials; its
 *                 contents need no initialization and are garbage afterwards.
 *
 * A sequence of at most pkv_decode_single_pass_max() tokens is attended by one workgroup per
 * head.  When max_context_len exceeds that bound, longer sequences are split into partitions
 * of pkv_decode_partition_tokens(...) tokens, each attended by its own workgroup, and a second
 * kernel merges the partial (max, sum, output) triples.  The split depends only on the length
 * and (desc, num_seqs, max_context_len), and the reduction order only on logical token order,
 * so results are bit-identical run to run, for any physical placement of the blocks, and for
 * any work-item order (pkv_paged_attention_decode_scheduled).
 *
 * A block id outside [0, num_blocks) in a block table is never dereferenced: that
 * (sequence, head) output is set to NaN instead.
 * Returns PKV_EINVAL (null pointers, negative sizes, workspace too small: PKV_ENOMEM),
 * PKV_EUNSUPPORTED, PKV_EHIP or PKV_OK.
 */
size_t pkv_decode_workspace_bytes(const pkv_cache_desc_t* desc, int32_t num_seqs,
                                  int32_t max_context_len);
int32_t pkv_decode_partition_tokens(const pkv_cache_desc_t* desc, int32_t num_seqs,
                                    int32_t max_context_len); /* 0: single pass, no split */
int32_t pkv_decode_single_pass_max(void);
pkv_status_t pkv_paged_attention_decode(const pkv_cache_desc_t* desc, void* out, const void* q,
                                        const void* k_pool, const void* v_pool,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t max_context_len, float scale, void* workspace,
                                        size_t workspace_bytes, pkv_stream_t stream);

/* The same attention with a host-built schedule: one workgroup per (work item, head) instead
 * of one per (sequence, possible partition, head), so no workgroup is launched for a
 * partition that does not exist and the longest work can be dispatched first.
 *
 * pkv_decode_schedule (host only) fills items (host out, `capacity` entries) with one entry
 * per (sequence s, partition p) that the lengths `lens` (host, num_seqs entries, the values
 * that will be in context_lens) produce under max_context_len, encoded s | p << 20, sorted
 * by decreasing token count (ties in (s, p) order); a length-0 sequence gets one item.
 * Returns the number of items, or -1 for bad arguments, capacity too small, num_seqs >= 2^20
 * or more than 2^11 partitions per sequence.
 * pkv_decode_schedule_grouped does the same but keeps sequences with equal group_keys (host,
 * num_seqs entries; e.g. each sequence's first physical block, equal for sequences that share
 * a prefix) adjacent: groups are ordered by their longest item, and inside a group items go
 * partition by partition, so the members read their shared blocks at the same time.
 * pkv_paged_attention_decode_scheduled takes those items in device memory (work_items,
 * num_items).  The items must be built from the same lengths as context_lens: a partition
 * left out leaves its output undefined (the kernels still stay inside every buffer); an item
 * naming a sequence or partition outside the call is ignored.
 * flags: 0, or PKV_DECODE_SHARED_KV when sequences of the batch share blocks -- K/V are then
 * read with ordinary (cache-allocating) loads so a block shared by a group is fetched from
 * HBM once, instead of the nontemporal loads used for K/V read by one sequence only.
 * Outputs are bit-identical to pkv_paged_attention_decode's for any item order and flags. */
#define PKV_DECODE_SHARED_KV 1u
int32_t pkv_decode_schedule(const pkv_cache_desc_t* desc, const int32_t* lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t* items, int32_t capacity);
int32_t pkv_decode_schedule_grouped(const pkv_cache_desc_t* desc, const int32_t* lens,
                                    const int32_t* group_keys, int32_t num_seqs,
                                    int32_t max_context_len, int32_t* items, int32_t capacity);
pkv_status_t pkv_paged_attention_decode_scheduled(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len, float scale,
    const int32_t* work_items, int32_t num_items, uint32_t flags, void* workspace,
    size_t workspace_bytes, pkv_stream_t stream);

/* XCD-weighted dealing of attention units (host only; what the step driver's attention
 * launches use, see "XCD balance" below).  The GPU deals workgroup b to XCD b % 8.  With a
 * split P in 1..1023, the units u = item * num_heads + head (longest work first) are dealt so
 * that the even XCDs receive unit u iff floor((u + 1) P / 1024) > floor(u P / 1024) -- a
 * share P / 1024 of every stretch of the list -- each half in list order, spread over its four
 * XCDs in turn.  pkv_decode_xcd_grid(units, P) is the number of workgroups such a launch takes
 * (units itself for P = 0, the identity deal); pkv_decode_xcd_slot_unit(slot, units, P) the
 * unit workgroup `slot` runs, or -1 for a slot with nothing to do.  Every unit goes to exactly
 * one slot.  Both return -1 / -2 for bad arguments (negative sizes, P outside 0..1023, slot
 * outside the grid).  Outputs do not depend on the deal. */
int64_t pkv_decode_xcd_grid(int64_t units, int32_t split);
int64_t pkv_decode_xcd_slot_unit(int64_t slot, int64_t units, int32_t split);
/* The split the stand-alone decode calls (pkv_paged_attention_decode, _scheduled, _noalloc) on
 * the current device deal their units with: 0 (evenly) until a step driver on the device has
 * measured one (see "XCD balance" below), which then applies to them too, or until
 * pkv_decode_set_xcd_split sets it (0..1023; PKV_EINVAL otherwise).  pkv_decode_xcd_split
 * returns it. */
pkv_status_t pkv_decode_set_xcd_split(int32_t split);
int32_t pkv_decode_xcd_split(void);

/* The same attention as pkv_paged_attention_decode, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument, and nothing is allocated by the call.  The split-context
 * partials go to a scratch array of PKV_DECODE_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds in each GPU's memory until the process ends.  A call whose partials need more than
 * that (pkv_decode_workspace_bytes(desc, num_seqs, max_context_len) after the clamp to
 * max_blocks_per_seq * block_size) returns PKV_ENOMEM before any device call.  Every call on
 * one GPU shares that GPU's array and leaves its contents behind (no call relies on them):
 * two such calls whose launches overlap on one GPU (on different streams) race and must be
 * ordered by the caller.  Arguments, results and other errors are those of
 * pkv_paged_attention_decode; PKV_EHIP also when the array's device address cannot be
 * obtained. */
#define PKV_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status_t pkv_paged_attention_decode_noalloc(const pkv_cache_desc_t* desc, void* out,
                                                const void* q, const void* k_pool,
                                                const void* v_pool, const int32_t* block_tables,
                                                int32_t max_blocks_per_seq,
                                                const int32_t* context_lens, int32_t num_seqs,
                                                int32_t max_context_len, float scale,
                                                pkv_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Multi-query paged attention: several new tokens of each sequence at once.
 * ("PagedAttention: Efficient LLM Serving with vLLM", "Advanced Features" -> "Prefix
 * Caching": a request whose prompt prefix is cached only computes the rest of its prompt;
 * same page, "Speculative Decoding Integration": draft tokens checked by the target model;
 * "The PagedAttention Algorithm", step 5: keys and values are gathered through the block
 * table.)
 *
 * Sequence s holds L_s = context_lens[s] tokens in the cache (clamped to max_context_len and
 * to max_blocks_per_seq * block_size); the last n_s = query_start[s+1] - query_start[s] of
 * them are its new tokens, whose K/V must already be in their slots (pkv_reshape_and_cache).
 * New token i (q row query_start[s] + i) sits at position P = L_s - n_s + i and attends to
 * positions 0 .. P only:
 *     out[query_start[s] + i][h] = softmax_t(scale * <q[query_start[s] + i][h], K_t>) V_t,
 *                                  t = 0 .. P, K_t, V_t read through block_tables[s]
 * A sequence with n_s = 1 is single-query decode; n_s = 0 contributes no rows.
 *
 *   out, q        device, [num_tokens][num_heads][head_dim], dtype, contiguous, 16-byte
 *                 aligned; out is written, q is read
 *   k_pool,v_pool device, pool layout above, 16-byte aligned; read only
 *   block_tables  device, int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  device, int32 [num_seqs]
 *   query_start   device, int32 [num_seqs + 1], nondecreasing from 0 to num_tokens; a
 *                 sequence whose rows fall outside [0, num_tokens) is skipped (rows untouched)
 *   max_query_len host: at least every n_s (rows of a longer sequence past it stay unwritten)
 *   scale         host; the softmax temperature, finite and > 0
 *   work_items    NULL (one workgroup per sequence, head and tile of pkv_multi_query_tile()
 *                 new tokens up to max_query_len), or device items from
 *                 pkv_multi_query_schedule (num_items of them)
 * Storage types f16 and bf16 only (the products run on 16-bit matrix-core instructions):
 * PKV_EUNSUPPORTED for f32.  Scores and outputs accumulate in fp32; the probabilities enter
 * the second product as fp16 (f16), or as a bf16 pair hi + lo (bf16).  A block id outside
 * [0, num_blocks) among a tile's keys is never dereferenced: that tile's outputs are NaN; so
 * are the rows of a sequence with n_s > L_s.  Returns PKV_EINVAL (null or misaligned
 * pointers, negative sizes, a scale that is not finite and positive, bad num_items),
 * PKV_EUNSUPPORTED (also for num_seqs * max_blocks_per_seq >= 2^32), PKV_EHIP or PKV_OK.
 *
 * pkv_multi_query_tile(): new tokens per workgroup tile (128: 8 waves of 16).
 * pkv_multi_query_schedule (host only): one item per (sequence s, tile of
 * pkv_multi_query_tile() new tokens) from host copies of query_start and context_lens,
 * encoded s | tile << 20; sequences that read the most keys first, a sequence's tiles
 * adjacent (the one reading the most keys first) so they share its K/V in L2.  Returns the
 * number of items, or -1 for bad arguments, capacity too small, a decreasing query_start,
 * num_seqs > 2^20 or more than 2^11 tiles per sequence.  Outputs are bit-identical for any
 * item order.  A device item naming a sequence or tile outside the call is ignored.
 * pkv_multi_query_schedule_grouped (host only): the same items, with group_keys (host,
 * [num_seqs], or NULL for the order above): sequences with equal keys -- for instance the
 * first physical block of their tables, so sequences that share prefix blocks after a
 * prefix-cache hit ("Advanced Features" -> "Prefix Caching") -- are scheduled side by side,
 * so their shared K/V is read from L2 while they run; groups that read the most keys first,
 * inside a group the order above.  Same return values.
 *
 * pkv_multi_query_schedule_packed (host only): tiles that pack the new tokens of
 * consecutive sequences sharing prefix blocks ("Advanced Features" -> "Prefix Caching", and
 * "KV-Cache Sharing") into full tiles of pkv_multi_query_tile() rows, for
 * pkv_paged_attention_multi_query_packed.  A run is a stretch of consecutive sequences with
 * new tokens whose tables (host copy, int32 [num_seqs][max_blocks]) hold the same first
 * `pre` keys in the same blocks, before every member's first new token; pre is a whole
 * number of 64-key stages, at least one, fixed by the run's first two members (a sequence
 * sharing fewer keys starts a new run).  Each tile is four int32: {sa, sb, first, pre}: rows
 * query_start[sa] + first onward, at most pkv_multi_query_tile() of them, through sequence sb
 * (pre = 0 and sa = sb outside runs).  Runs that read the most keys first, a run's tiles
 * adjacent.  tiles: host, int32 [capacity][4]; a capacity of num_seqs *
 * ceil(max new tokens / pkv_multi_query_tile()) always suffices.  Returns the number of
 * tiles, or -1 for bad arguments (null pointers, max_blocks or block_size <= 0, a
 * decreasing query_start) or too small a capacity.
 * pkv_paged_attention_multi_query_packed: pkv_paged_attention_multi_query over such tiles
 * (tiles: device, int32 [num_tiles][4], 16-byte aligned).  Per tile and head, a workgroup
 * stages the shared keys once for all its rows and then each member's own keys for that
 * member's rows, so tiles are full where sequences share a prompt.  The kernel re-checks on
 * the device that every member's table holds the tile's first pre keys in the same blocks
 * and that they precede every member's new tokens, and otherwise reads each member's keys on
 * its own: for tiles that cover every new token once (the schedule's do), the outputs are
 * those of pkv_paged_attention_multi_query bit for bit (every row sees the same keys in the
 * same 64-key stages; a step a row does not see adds exact zeros).  A tile naming sequences outside
 * the call, a negative first or a pre that is not a whole number of stages is ignored.  Same
 * other arguments and returns; PKV_EINVAL also for num_tiles < 0 or null or misaligned tiles
 * with num_tiles > 0.
 */
int32_t pkv_multi_query_tile(void);
int32_t pkv_multi_query_schedule(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_context_len, int32_t* items,
                                 int32_t capacity);
int32_t pkv_multi_query_schedule_grouped(const int32_t* query_start,
                                         const int32_t* context_lens, const int32_t* group_keys,
                                         int32_t num_seqs, int32_t max_context_len,
                                         int32_t* items, int32_t capacity);
pkv_status_t pkv_paged_attention_multi_query(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale,
    const int32_t* work_items, int32_t num_items, pkv_stream_t stream);
int32_t pkv_multi_query_schedule_packed(const int32_t* query_start,
                                        const int32_t* context_lens,
                                        const int32_t* block_tables, int32_t max_blocks,
                                        int32_t block_size, int32_t num_seqs,
                                        int32_t max_context_len, int32_t* tiles,
                                        int32_t capacity);
pkv_status_t pkv_paged_attention_multi_query_packed(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale,
    const int32_t* tiles, int32_t num_tiles, pkv_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Append new tokens' keys and values to the cache.
 * ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
 * step 2: generated tokens fill the current block.)
 *
 * For every i < num_tokens with slot = slot_mapping[i] in [0, num_blocks * block_size):
 *     k_pool[slot / block_size][h][slot % block_size][:] = k[i][h][:]   for every head h
 * and the same for v.  A byte copy: bit-exact, NaN payloads included.  A negative slot, or
 * one at or past num_blocks * block_size, writes nothing.  Slots in one call must be
 * distinct (two tokens writing one slot leave either value).
 *
 *   k, v          device, [num_tokens][num_heads][head_dim], dtype, contiguous
 *   k_pool,v_pool device, pool layout above; written
 *   slot_mapping  device, int32 [num_tokens]
 */
pkv_status_t pkv_reshape_and_cache(const pkv_cache_desc_t* desc, const void* k, const void* v,
                                   void* k_pool, void* v_pool, const int32_t* slot_mapping,
                                   int32_t num_tokens, pkv_stream_t stream);

/* Host check of that precondition, for a caller that holds the slots in host memory (the step
 * driver runs it on every step's slots before they are uploaded; the binding runs it on a
 * host copy when PKV_DEBUG=1 is set in the environment): PKV_EINVAL if two slots in
 * [0, num_blocks * block_size) are equal (slots outside that range are skipped by the kernel
 * and ignored here), else PKV_OK.  slot_mapping: host, int32 [num_tokens]. */
pkv_status_t pkv_check_slot_mapping(const pkv_cache_desc_t* desc, const int32_t* slot_mapping,
                                    int32_t num_tokens);

/* ---------------------------------------------------------------------------------------
 * Copy whole blocks, in every layer, for copy-on-write of shared prefix blocks.
 * ("PagedAttention: Efficient LLM Serving with vLLM", "Advanced Features" ->
 * "KV-Cache Sharing (Copy-on-Write)": blocks stay shared until a write, as the memory pages
 * of a forked process do.)
 *
 * For every layer l < num_layers and pair p < num_pairs with (src, dst) = (pairs[2p],
 * pairs[2p+1]):  k_pools[l][dst] = k_pools[l][src] and v_pools[l][dst] = v_pools[l][src]
 * (one block = num_heads * block_size * head_dim elements).  Bit-exact.  A pair with src or
 * dst outside [0, num_blocks) is skipped.  Destinations must be distinct and no destination
 * may be a source in the same call (the block manager only produces such pairs).
 *
 *   k_pools,v_pools host arrays of num_layers device pointers, each a pool of shape `desc`
 *   pairs           device, int32 [num_pairs][2]
 */
pkv_status_t pkv_copy_blocks(const pkv_cache_desc_t* desc, void* const* k_pools,
                             void* const* v_pools, int32_t num_layers, const int32_t* pairs,
                             int32_t num_pairs, pkv_stream_t stream);

/* Host check of those preconditions (run by the step driver on every step's pairs before
 * they are uploaded, and by the binding on a host copy when PKV_DEBUG=1): PKV_EINVAL if,
 * among the pairs whose src and dst are both in [0, num_blocks), a destination repeats or is
 * also a source; else PKV_OK.  pairs: host, int32 [num_pairs][2]. */
pkv_status_t pkv_check_copy_pairs(const pkv_cache_desc_t* desc, const int32_t* pairs,
                                  int32_t num_pairs);

/* ---------------------------------------------------------------------------------------
 * Copy blocks between two pools of the same shape -- out of HBM into a pinned host swap pool
 * and back -- for preemption by swapping ("PagedAttention: Efficient LLM Serving with vLLM",
 * "vLLM: The Serving Engine": swap the KV cache to CPU memory when the GPU is full and resume
 * later; the aipaper.jasonlin.tech page, "Key contributions": with small blocks, swapping
 * means many small transfers).
 *
 * For every layer l and pair p with (src, dst) = (pairs[2p], pairs[2p+1]):
 *     dst_k[l][dst] = src_k[l][src] and dst_v[l][dst] = src_v[l][src]     (bit-exact)
 * All pairs of all layers are copied by one kernel launch (per 64 layers), not one transfer per
 * block.  Each pool pointer, and pairs, may be device memory or pinned host memory
 * (hipHostMalloc; e.g. a torch pin_memory tensor), which the kernel reaches over PCIe; pageable
 * host memory is refused (PKV_EINVAL).  The descriptors must agree in everything but
 * num_blocks.  A pair with src outside [0, src num_blocks) or dst outside [0, dst num_blocks)
 * is skipped.  Destinations must be distinct.
 *   src_k/src_v/dst_k/dst_v  host arrays of num_layers pool pointers
 *   pairs                    int32 [num_pairs][2], device or pinned host memory
 */
pkv_status_t pkv_swap_blocks(const pkv_cache_desc_t* src_desc, const pkv_cache_desc_t* dst_desc,
                             const void* const* src_k, const void* const* src_v,
                             void* const* dst_k, void* const* dst_v, int32_t num_layers,
                             const int32_t* pairs, int32_t num_pairs, pkv_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Host block manager: on-demand allocation, reference counts, copy-on-write decisions.
 * Plain C++, no device calls; one instance is used by one thread.
 * ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
 * steps 1-4 and "Memory Efficiency"; "Advanced Features" -> "KV-Cache Sharing
 * (Copy-on-Write)".)
 *
 * Policy: free blocks are handed out from a free list whose initial order is `free_order`
 * (host, a permutation of 0..num_blocks-1; NULL = ascending ids); a freed block goes on top
 * of the list and is handed out next.  free_seq returns a sequence's blocks so that its
 * logical block 0 is on top.
 *   add_seq(seq, len)     new sequence with ceil(len / block_size) blocks
 *   fork(parent, child)   child shares every block of parent (each gains a reference)
 *   append_slot(seq)      room for one more token: a new block when the last one is full;
 *                         if the target block is shared (reference count > 1) a fresh block
 *                         replaces it in this sequence's table and (src, dst) is reported
 *                         for pkv_copy_blocks; the last holder writes in place.
 *   free_seq(seq)         drop one reference from each block; blocks at zero are freed
 *   add_seq_cached(seq, tokens, len)  prefix cache ("Advanced Features" -> "Prefix Caching":
 *                         cached prefix blocks are reused by later requests): a full prompt
 *                         block is keyed by its block_size token ids and the key of the block
 *                         before it; the leading full blocks found in the cache are shared
 *                         (one more reference each), the rest are fresh and the fresh full
 *                         blocks are entered in the cache (the caller fills their K/V before
 *                         any later lookup relies on them).  *cached_tokens = tokens whose K/V
 *                         is already present.  The trailing partial block is never cached.
 *                         A cached block whose last reference goes is parked, not freed;
 *                         blocks come from the plain free list first, then by evicting the
 *                         block parked longest ago (which leaves the cache).
 * num_free counts plain free and parked blocks.
 * Errors: PKV_EINVAL for an unknown or duplicate sequence id or a null argument;
 * PKV_ENOMEM when the pool has no free block -- the state is then left unchanged.
 * ---------------------------------------------------------------------------------------*/
typedef struct pkv_alloc pkv_alloc_t;

pkv_alloc_t* pkv_alloc_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* free_order /* host, may be NULL */);
void pkv_alloc_destroy(pkv_alloc_t* a);
pkv_status_t pkv_alloc_add_seq(pkv_alloc_t* a, int64_t seq, int32_t len);
pkv_status_t pkv_alloc_fork(pkv_alloc_t* a, int64_t parent, int64_t child);
/* slot: host out; cow_src / cow_dst: host out, -1 when no copy is needed. */
pkv_status_t pkv_alloc_append_slot(pkv_alloc_t* a, int64_t seq, int32_t* slot, int32_t* cow_src,
                                   int32_t* cow_dst);
/* append_slot for seqs[0..n-1] in order; slots[i] (host out, n entries) receives each slot;
 * cow_pairs (host out, room for 2*n int32) receives the (src, dst) pairs in order and
 * *num_cow their count; *num_done the number of sequences served -- processing stops at
 * the first error, which is returned. */
pkv_status_t pkv_alloc_append_slots(pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                                    int32_t* slots, int32_t* cow_pairs, int32_t* num_cow,
                                    int32_t* num_done);
/* The number of blocks append_slots(seqs[0..n-1]) would take from the pool -- one per sequence
 * that starts a new block, one per copy-on-write of a shared block -- into *blocks (host
 * out), without changing anything; the same sequence may be listed more than once.  A
 * scheduler compares it with pkv_alloc_num_free to decide, before a step, whether to preempt
 * ("vLLM: The Serving Engine").  PKV_EINVAL for an unknown sequence or a null argument. */
pkv_status_t pkv_alloc_append_need(const pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                                   int32_t* blocks);
pkv_status_t pkv_alloc_free_seq(pkv_alloc_t* a, int64_t seq);
/* Batched forms for a scheduler that starts, forks (beam search, parallel sampling: "KV-Cache
 * Sharing (Copy-on-Write)") or ends many sequences per step with one host call each:
 * add_seq(seqs[i], lens[i]), fork(parents[i], children[i]) and free_seq(seqs[i]) for
 * i = 0..n-1 in order (host arrays).  Processing stops at the first error, which is returned;
 * *num_done (host out) is the number of calls that succeeded, whose effects stay. */
pkv_status_t pkv_alloc_add_seqs(pkv_alloc_t* a, const int64_t* seqs, const int32_t* lens,
                                int32_t n, int32_t* num_done);
pkv_status_t pkv_alloc_fork_many(pkv_alloc_t* a, const int64_t* parents, const int64_t* children,
                                 int32_t n, int32_t* num_done);
pkv_status_t pkv_alloc_free_seqs(pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                                 int32_t* num_done);
/* Copies up to `cap` physical block ids of seq's table into out (host); *n = table length. */
pkv_status_t pkv_alloc_block_table(const pkv_alloc_t* a, int64_t seq, int32_t* out, int32_t cap,
                                   int32_t* n);
/* Fills a dense host int32 [n][max_blocks] table (unused entries -1) and int32 [n] lengths
 * for seqs[0..n-1]; PKV_EINVAL if a table is longer than max_blocks. */
pkv_status_t pkv_alloc_export(const pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t* tables, int32_t* lens);
int32_t pkv_alloc_seq_len(const pkv_alloc_t* a, int64_t seq); /* -1 if unknown */
int32_t pkv_alloc_num_free(const pkv_alloc_t* a);
pkv_status_t pkv_alloc_add_seq_cached(pkv_alloc_t* a, int64_t seq, const int32_t* tokens,
                                      int32_t len, int32_t* cached_tokens);
int32_t pkv_alloc_num_cached(const pkv_alloc_t* a); /* blocks in the prefix cache */
/* Preemption by swapping ("PagedAttention: Efficient LLM Serving with vLLM", "vLLM: The
 * Serving Engine": swap the KV cache to CPU memory when the GPU is full, resume later).
 * Moves sequences seqs[0..n-1] from block manager `from` to block manager `to` (same
 * block_size; e.g. the HBM pool's and a pinned host pool's): each distinct block they use gets
 * one block of `to` in first-use order (a block shared among them stays shared), tables and
 * lengths move over, `from` drops their references, and the (block in from, block in to)
 * pairs go to pairs (host out, room for 2 * capacity int32) for pkv_swap_blocks.
 * PKV_EINVAL if a sequence is unknown in `from`, already in `to`, listed twice, or shares a
 * block with a sequence not in the list (move the whole group), or capacity is too small;
 * PKV_ENOMEM if `to` has too few free blocks.  On error nothing changes. */
pkv_status_t pkv_alloc_move_seqs(pkv_alloc_t* from, pkv_alloc_t* to, const int64_t* seqs,
                                 int32_t n, int32_t* pairs, int32_t capacity,
                                 int32_t* num_pairs);
int32_t pkv_alloc_refcount(const pkv_alloc_t* a, int32_t block); /* -1 if out of range */
/* Unused slots of blocks in use: per block, block_size minus the most tokens any sequence
 * keeps in it ("Memory Efficiency": 100 tokens in 16-token blocks waste 12 slots). */
int64_t pkv_alloc_wasted_slots(const pkv_alloc_t* a);


/* ---------------------------------------------------------------------------------------
 * Decode-step driver: one decode iteration of a batch over every layer, in one call.
 * ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
 * steps 1-5: extend each sequence's blocks on demand, fill the new slot, keep the page table,
 * attend through it; "Advanced Features" -> "KV-Cache Sharing (Copy-on-Write)".)
 *
 * pkv_stepper_step(seqs[0..n-1]) does, in order:
 *   1. pkv_alloc_append_slots on the stepper's block manager (one new slot per sequence),
 *      then exports the dense block tables and lengths, into a pinned host staging area
 *      (eight areas used in turn, so the host can prepare later steps while step i runs);
 *   2. one prologue kernel on `stream` pulls the packed index data from the pinned area (over
 *      PCIe) into an area of d_index and, when there are no copy-on-write pairs, also
 *      appends the first layer's new K/V:
 *      int32 tables [n][max_blocks_per_seq] | lens [n] | slots [n] | cow pairs [num_cow][2] |
 *      decode work items [num_items] -- longest work first (pkv_decode_schedule) or, when
 *      sequences share their first block, grouped by it (pkv_decode_schedule_grouped) and
 *      decoded with PKV_DECODE_SHARED_KV;
 *   3. pkv_copy_blocks over every layer when there are copy-on-write pairs;
 *   4. for each layer l: pkv_reshape_and_cache(k_new[l], v_new[l] -> pools[l]) (done by the
 *      prologue for layer 0 when there was no copy), then
 *      pkv_paged_attention_decode_scheduled(q[l] -> out[l]) with the lengths including the
 *      new token -- or, when sequences share their first blocks (parallel sampling, beam
 *      search, a cached prompt: "Advanced Features" -> "KV-Cache Sharing"), the cache is f16
 *      or bf16, q and out are 16-byte aligned, no context exceeds 4096 tokens, the packed
 *      tiles (pkv_multi_query_schedule_packed, one new token per sequence) hold two sequences
 *      or more on average and number at least 448 / num_heads, the same attention through
 *      pkv_paged_attention_multi_query_packed, which stages each group's shared blocks once
 *      for all its members (the index area then holds query_start [n + 1] and the tiles
 *      after the pairs).  pkv_stepper_last_attention tells which ran (PKV_STEP_ATTN_*; -1
 *      before any step and after a step with n = 0).
 * Everything after step 1 is asynchronous on `stream`.
 *
 * Errors.  Before step 1 the call makes every check pkv_stepper_check makes (below) and
 * returns its error, if any, with nothing changed: the block manager, the pools, the staging
 * areas and the device index area are as before, nothing is launched and *num_done is 0.  So
 * the pool running out (PKV_ENOMEM), an unknown or repeated sequence, a context that outgrows
 * max_blocks_per_seq (PKV_EINVAL) or a workspace too small for the split-context partials of
 * this step's longest context (PKV_ENOMEM) are reported before any sequence is extended.
 * After step 1 the slots and copy pairs about to be uploaded are checked with
 * pkv_check_slot_mapping and pkv_check_copy_pairs; a failure there (PKV_EINVAL) would mean the
 * block manager broke its own invariants: the sequences are then extended but nothing is
 * launched.  Only PKV_EHIP (a launch the runtime refused) can come back after a launch.
 *
 * pkv_stepper_check(alloc, desc, max_seqs, max_blocks_per_seq, seqs, n, io, workspace,
 * workspace_bytes, max_len) makes the checks of a step of a stepper created with
 * (alloc, desc, max_seqs, max_blocks_per_seq), host only, without changing anything: the
 * descriptor; n <= max_seqs; the io pointers (non-null; pools and new K/V 16-byte aligned;
 * scale finite); every sequence known and listed once; each one's length after the append
 * within max_blocks_per_seq * block_size; the blocks the append takes
 * (pkv_alloc_append_need) within pkv_alloc_num_free; the attention grid within its limits;
 * the workspace >= pkv_decode_workspace_bytes(desc, n, longest context after the append)
 * and 16-byte aligned.  *max_len (host out) receives that longest context.
 *
 * Streams.  Steps may be issued on different streams: when a step's stream differs from the
 * previous step's, the new stream first waits for everything the previous stream had queued
 * (an event of the stepper's own), since the two steps share the staging areas, the device
 * index area and the split-context workspace.
 *
 * The stepper allocates only pinned host memory (staging areas, calibration stamps) and HIP
 * events of its own; the caller owns the device buffer d_index (pkv_stepper_index_bytes
 * bytes, 16-byte aligned: eight areas used by the steps in turn) and the workspace.  The
 * host refills a staging area only after the prologue that read it (eight launches earlier)
 * is known to have finished: every seventh prologue launch records its own completion marker
 * (no event packet sits between kernels, and the few microseconds of idle GPU a marked
 * launch leaves behind it come once every seven steps), and the host waits for the oldest
 * marker at or after that prologue.  pkv_stepper_last_index returns the device address of
 * the packed index data of the last step.  pkv_stepper_destroy waits until the stepper's
 * prologues are done with the staging areas before freeing them (it records an event on the
 * stream of the last step), so destroy the stepper before that stream.
 * attn_events: NULL, or a host array of 2 * num_layers hipEvent_t (created with timing): event
 * 2l takes the start and event 2l+1 the end of layer l's attention launch, recorded by the
 * launch itself (hipExtLaunchKernel) so that no event packet sits between kernels; a step with
 * n = 0 records them back to back on `stream`.
 *
 * XCD balance.  The eight XCDs of an MI355X do not stream K/V equally fast (measured: the odd
 * ones take ~10% longer per token), so an even deal of the units leaves the fast half idle at
 * the end of every attention launch.  The stepper measures the two halves on the first step
 * with at least 1536 units (enough to fill the chip twice; a smaller launch does not load the
 * halves enough to tell them apart): that step's layer-0 attention launch deals unit b to
 * workgroup b and each workgroup leaves its duration, XCD, token count and start tick in
 * pinned host memory of the stepper's own; a later step reads them once that launch is done
 * (never waiting for it), keeps the workgroups that ended before the first XCD ran out of
 * work, and from then on every attention launch deals the units with the split
 * P = 1024 * speed(even) / (speed(even) + speed(odd)), bounded to 384..640
 * (pkv_decode_xcd_grid / _slot_unit above).
 * P stays 0 (no weighting) when the halves differ by less than 1%, when the hardware does not
 * place workgroup b on XCD b % 8, or after four measuring launches without enough workgroups
 * per half.
 * pkv_stepper_xcd_split returns the split in use (0: none; -1 for a null stepper);
 * pkv_stepper_set_xcd_split fixes it (0..1023, 0: none) and stops the measurement, or with -1
 * starts a new measurement on the next step (PKV_EINVAL otherwise).  pkv_stepper_xcd_rates
 * gives the last measurement (host outs): each half's tokens per 100 MHz tick of workgroup
 * time (0 until measured) and its outcome, a PKV_XCD_* value.  Outputs do not depend on the
 * split.
 * ---------------------------------------------------------------------------------------*/
typedef struct pkv_stepper pkv_stepper_t;

typedef struct {
  int32_t num_layers;
  void* const* k_pools;      /* host arrays [num_layers] of device pools (layout above) */
  void* const* v_pools;
  const void* const* q;      /* host arrays [num_layers] of device [n][num_heads][head_dim] */
  const void* const* k_new;
  const void* const* v_new;
  void* const* out;
  float scale;
} pkv_layer_io_t;

size_t pkv_stepper_index_bytes(const pkv_cache_desc_t* desc, int32_t max_seqs,
                               int32_t max_blocks_per_seq);
pkv_stepper_t* pkv_stepper_create(pkv_alloc_t* alloc, const pkv_cache_desc_t* desc,
                                  int32_t max_seqs, int32_t max_blocks_per_seq, void* d_index);
void pkv_stepper_destroy(pkv_stepper_t* st);
pkv_status_t pkv_stepper_step(pkv_stepper_t* st, const int64_t* seqs, int32_t n,
                              const pkv_layer_io_t* io, void* workspace, size_t workspace_bytes,
                              void* const* attn_events, int32_t* max_len, int32_t* num_cow,
                              int32_t* num_done, pkv_stream_t stream);
const void* pkv_stepper_last_index(const pkv_stepper_t* st);
int32_t pkv_stepper_last_attention(const pkv_stepper_t* st);
#define PKV_STEP_ATTN_DECODE 0       /* pkv_paged_attention_decode_scheduled */
#define PKV_STEP_ATTN_MULTI_QUERY 1  /* pkv_paged_attention_multi_query_packed */
int32_t pkv_stepper_xcd_split(const pkv_stepper_t* st);
pkv_status_t pkv_stepper_set_xcd_split(pkv_stepper_t* st, int32_t split);
#define PKV_XCD_NONE 0       /* nothing measured (yet) */
#define PKV_XCD_IN_FLIGHT 1  /* the stamped launch has not finished */
#define PKV_XCD_MEASURED 2   /* rates measured, split set from them */
#define PKV_XCD_TOO_FEW 3    /* the last stamped launch had too few workgroups per half */
#define PKV_XCD_UNMAPPED 4   /* workgroup b did not run on XCD b % 8: no weighting */
#define PKV_XCD_FAILED 5     /* the runtime reported an error on the stamped launch */
pkv_status_t pkv_stepper_xcd_rates(const pkv_stepper_t* st, double* even, double* odd,
                                   int32_t* outcome);
/* The measurement itself, host only: from `units` stamps of a launch that dealt unit b to
 * workgroup b (4 uint32 each: duration in 100 MHz ticks, XCD | 0x100 for a workgroup that
 * attended tokens, tokens, low 32 bits of its start tick), the split the stepper would take:
 * -1 when too few workgroups per half ended before the first XCD ran out of work, 0 when
 * workgroup b did not run on XCD b % 8 or the halves differ by less than 1%, else 384..640.
 * even / odd / outcome (host outs) as pkv_stepper_xcd_rates gives them.  -2 for bad
 * arguments. */
int32_t pkv_xcd_split_from_stamps(const uint32_t* stamps, int64_t units, double* even,
                                  double* odd, int32_t* outcome);
pkv_status_t pkv_stepper_check(const pkv_alloc_t* alloc, const pkv_cache_desc_t* desc,
                               int32_t max_seqs, int32_t max_blocks_per_seq, const int64_t* seqs,
                               int32_t n, const pkv_layer_io_t* io, const void* workspace,
                               size_t workspace_bytes, int32_t* max_len);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
