/*
 * lra.h - attention over a shared-base + low-rank KV cache on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (LRAgent: Efficient KV Cache Sharing for Multi-LoRA LLM
 * Agents, abstract; PReCache abstract and Figure 1 caption): every cached
 * key and value is the sum of a base part computed with the pretrained
 * weights, shared by all agents, and an adapter part kept in its low-rank
 * form,
 *
 *     K[n] = K_base[n] + rope_n(L_k[n] . B_k)      V[n] = V_base[n] + L_v[n] . B_v
 *
 * with L = X . A the low-rank cache of the hidden states X and (A, B) the
 * LoRA factors of the key/value projections. The full-dimension adapter
 * term is never written to device memory: keys are rebuilt per tile in
 * registers, and the value term is applied once per output row as
 * (P . L_v) . B_v (LRAgent abstract: the kernel reorders the attention
 * computation so the low-rank cache is not expanded to full dimension).
 *
 * Conventions shared by every entry point
 * - All pointers are device pointers unless marked (host).
 * - The caller owns every buffer. The library allocates nothing, keeps no
 *   pointer after it returns and has no state other than a thread-local
 *   error message. Work is enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream) and the call returns without waiting; buffers must stay
 *   alive until that work has run.
 * - Return value: LRA_OK (0) or a negative lra_status. Argument checks run
 *   on the host before any HIP call; nothing throws or aborts. The message
 *   of the last failure on the calling thread is lra_last_error().
 * - Device-side contents (block ids, agent ids, lengths) are trusted: an
 *   out-of-range value is undefined behaviour. liblra_debug.so exports the
 *   same entry points over the same kernels, built with LRA_DEBUG_CHECKS:
 *   before each attention launch it checks on the device, for every
 *   sequence, the context length (1..max_context_len), the block ids of the
 *   used table entries (>= 0; the pool size is not passed, so not the upper
 *   bound), the agent id (-1..N_agents-1), that agent's rank
 *   (1..max_rank, a multiple of 8) and pool / B pointers,
 *   adapter_start (>= 0), the query count (0..min(max_q_len, context
 *   length)), the decode rows of a varlen call (cu_q_lens[s] = s for
 *   s <= S_dec), and that group_offsets rise
 *   from 0 to S with every sequence of a group sharing the first one's
 *   context length and block-table row. It synchronises `stream` to read
 *   the result and returns LRA_ERR_INVALID_ARG naming the first failing
 *   check before the attention kernels run (so it cannot be captured in a
 *   graph). For lr_cache_build and lr_cache_build_multi it checks, before the
 *   launch, that the workspace's tile counters are zero.
 * - dtype applies to every floating-point tensor of a call (q, pools,
 *   adapters, out; X, A, L for the cache build). Accumulation is fp32.
 *
 * Cache layout (block size 16 tokens, NB physical blocks):
 *   k_base   [NB, Hkv, 16, d]   keys of one (block, head), token-major
 *   v_base   [NB, Hkv, d, 16]   values of one (block, head), 16 tokens of a dim contiguous
 *   L_k pool [NB, r/8, 16, 8]   low-rank key rows in chunks of 8 ranks: rank j of
 *                               slot t at ((j/8)*16 + t)*8 + j%8 within the block
 *                               (ranks 8q..8q+7 of all 16 slots are one contiguous run)
 *   L_v pool [NB, r, 16]        rank-major low-rank value rows
 *   B_k, B_v [r, Hkv*d]         per agent; column h*d + i feeds KV head h, dim i
 * A sequence's token n lives in physical block block_tables[s][n/16], slot
 * n%16, in the base pools and in the low-rank pools of its agent alike.
 * Keys in k_base are stored after the rotary embedding; the adapter key
 * term is rotated at its absolute 0-based position n (rotate-half pairing
 * (i, i+d/2), angle n*rope_theta^(-2i/d)); values are not rotated.
 */
#ifndef LRA_H
#define LRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRA_VERSION 500

typedef enum lra_status {
  LRA_OK = 0,
  LRA_ERR_INVALID_ARG = -1, /* null pointer, bad size or misaligned buffer */
  LRA_ERR_UNSUPPORTED = -2, /* valid but not built: head dim, rank, dtype, GQA ratio */
  LRA_ERR_WORKSPACE = -3,   /* workspace smaller than the size query returned */
  LRA_ERR_LAUNCH = -4       /* the HIP runtime rejected a launch */
} lra_status;

typedef enum lra_dtype { LRA_F32 = 0, LRA_BF16 = 1 } lra_dtype;

/* Where lr_cache_build stores rows when a slot mapping is given. */
typedef enum lra_l_layout {
  LRA_L_TOKEN_MAJOR = 0, /* pool [NB, 16, ldl]: row of slot s at L + s*ldl (a plain paged row store) */
  LRA_L_RANK_MAJOR = 1,  /* pool [NB, n_cols, 16]: column c of slot s at L + ((s/16)*n_cols + c)*16 + s%16 (the L_v layout) */
  LRA_L_KEY_CHUNKED = 2  /* pool [NB, n_cols/8, 16, 8]: column c of slot s at
                            L + (s/16)*16*n_cols + ((c/8)*16 + s%16)*8 + c%8 (the L_k layout; n_cols % 8 == 0) */
} lra_l_layout;

/* LRA_VERSION of the built library. */
int lra_version(void);

/* Message of the last failed call on this thread ("" if none). Valid until
 * the next lra call on the same thread. */
const char* lra_last_error(void);

/* ------------------------------------------------------------------------
 * Low-rank cache build: L = X . A (PReCache abstract and Figure 1 caption:
 * an agent's compact low-rank cache is precomputed from the hidden states of
 * a context segment; LRAgent abstract: the adapter component is stored in
 * its low-rank form).
 *
 *   X [n_tokens, hidden] row stride ldx, A [hidden, n_cols] row stride lda.
 *   Products in fp32 from bf16 inputs, one fp32 sum per output, one
 *   round-to-nearest-even to bf16 at the store.
 *   slot_mapping == NULL: dense store, row i at L + i*ldl (token-major only).
 *   slot_mapping != NULL: int64 [n_tokens]; row i goes to slot
 *   slot_mapping[i] of a paged pool laid out as `l_layout` says; a negative
 *   slot skips the row. Columns [0, n_cols) of each row are written.
 *   dtype: LRA_BF16. hidden % 8 == 0, 1 <= n_cols <= 512, ldx, lda >= their
 *   widths, X 16-byte aligned with ldx % 8 == 0.
 *   workspace: lr_cache_build_workspace_size(...) bytes of device memory,
 *   16-byte aligned (0 bytes, and NULL allowed, when hidden <= 512). The
 *   hidden dimension is summed in slices of 512 by separate workgroups; the
 *   workspace holds their fp32 partial sums and, in its first 4096 bytes, one
 *   counter per output tile. Those 4096 bytes must be zero the first time a
 *   workspace is used (allocate it zero-filled); every call leaves them zero
 *   again, so the same workspace serves any later build of any size up to
 *   the one it was sized for. Calls that overlap in time must use different
 *   workspaces. The partial sums of a column are added in slice order, so a
 *   result does not depend on the order in which workgroups finish.
 * ---------------------------------------------------------------------- */
size_t lr_cache_build_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_cols);

int lr_cache_build(const void* X, int64_t ldx, const void* A, int64_t lda, void* L, int64_t ldl,
                   const int64_t* slot_mapping, int32_t l_layout, int32_t n_tokens, int32_t hidden,
                   int32_t n_cols, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Low-rank caches of several adapters from one pass over X (PReCache,
 * Figure 1 caption, A1-A3: the hidden states produced when a context
 * segment is first processed build the low-rank caches of every agent).
 * A holds the adapters' down-projections side by side: columns
 * [group_cols[g], group_cols[g+1]) form group g (say agent a's A_k, then its
 * A_v), of width r_g. Row i of X A, restricted to group g, goes to slot
 * slot_mapping[i] of the pool group_pools[g], laid out as group_layouts[g]
 * says with n_cols = r_g (token-major [NB,16,r_g], rank-major [NB,r_g,16] or
 * key-chunked [NB,r_g/8,16,8]);
 * a negative slot skips the row. Every column of X A is formed exactly as
 * lr_cache_build forms it (same sums in the same order), so each group's
 * rows are bit-identical to a separate lr_cache_build of that group, while X
 * is read once for all of them.
 *   group_cols (host) int32 [n_groups+1], group_cols[0] = 0, strictly
 *   increasing, group_cols[n_groups] = n_cols. group_pools (host) [n_groups]
 *   device pointers; group_layouts (host) int32 [n_groups] of lra_l_layout.
 *   1 <= n_groups <= 64. slot_mapping: int64 [n_tokens], required.
 *   Sizes, dtype and workspace as for lr_cache_build (the workspace query is
 *   lr_cache_build_workspace_size with the total n_cols; its first 4096 bytes
 *   zero-filled before first use).
 * ---------------------------------------------------------------------- */
int lr_cache_build_multi(const void* X, int64_t ldx, const void* A, int64_t lda, int32_t n_groups,
                         const int32_t* group_cols, void* const* group_pools, const int32_t* group_layouts,
                         const int64_t* slot_mapping, int32_t n_tokens, int32_t hidden, int32_t n_cols,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention: one query token per sequence at position T_s - 1 over
 * keys 0..T_s-1 (T_s = context_lens[s] includes the current token).
 *
 *   q, out        [S, Hq, d]; q already rotated. out[s, j] for query head j
 *                 reads KV head j / (Hq/Hkv). Hq a multiple of Hkv, at most 16
 *                 query heads per KV head, Hkv <= 65535 (LRA_ERR_UNSUPPORTED
 *                 beyond).
 *   block_tables  int32 [S, max_blocks]; entries past ceil(T_s/16) are not read.
 *   context_lens  int32 [S], 1 <= T_s <= max_blocks*16 and <= max_context_len.
 *   group_offsets int32 [num_groups+1] or NULL (every sequence its own group).
 *                 Sequences group_offsets[g] .. group_offsets[g+1]-1 must share
 *                 the block-table row and context length of the first one;
 *                 the base cache is then read once for all of them (the
 *                 shared base component of LRAgent's abstract). At most
 *                 min(8, 16 / (Hq/Hkv), 256 / r_pad) sequences of a group
 *                 share one pass (r_pad: max_rank rounded up to 16, 32 or 64);
 *                 larger groups are served in several passes, whose reads of
 *                 the base are placed on one XCD so that the later ones can
 *                 hit its L2.
 *   agent_ids     int32 [S], in [0, N_agents), or -1 for a sequence without
 *                 an adapter (it attends over the base cache alone; PReCache
 *                 Figure 1 caption batches such adapter-free paths with
 *                 adapted ones).
 *   adapter_start int32 [S] or NULL (all 0): the first token position of
 *                 sequence s that carries the adapter terms; tokens before it
 *                 keep the base key and value (the activation point of an
 *                 activated adapter: Efficient Multi-Adapter LLM Serving via
 *                 Cross-Model KV-Cache Reuse with Activated LoRA, abstract).
 *                 Cache blocks wholly before every start of a tile skip the
 *                 key rebuild, the low-rank loads and P L_v. Not read without
 *                 adapters. Any value is valid: <= 0 means every token, >= T_s none.
 *   l_k_pools, l_v_pools
 *                 device arrays [N_agents] of device pointers to each agent's
 *                 low-rank pools ([NB,16,r_a] and [NB,r_a,16]). Agents with
 *                 shared-A adapters pass the same pointers (LRAgent abstract:
 *                 shared-A lets the low-rank cache itself be shared).
 *   b_k, b_v      device arrays [N_agents] of device pointers to [r_a, Hkv*d].
 *                 b_k == NULL: the call has no key adapter (K = K_base; adapters
 *                 on q and v only, the setting PReCache's appendix Table 13
 *                 caption compares against); l_k_pools is then not read and
 *                 may be NULL, and no key is rebuilt. b_v == NULL likewise
 *                 for values (V = V_base, l_v_pools not read). Both NULL:
 *                 plain attention over the base cache; agent_ids, ranks and
 *                 N_agents are not read and max_rank must be 0.
 *   ranks         int32 [N_agents], each in 1..max_rank and a multiple of 8
 *                 (the L_k pool holds chunks of 8 ranks).
 *   max_rank      (host) 1..64, or 0 without adapters (pass the same value to
 *                 the workspace query). d: 64 or 128 (bf16: 128). block_size: 16.
 *   sm_scale      softmax scale (usually 1/sqrt(d)).
 *   rope_theta    rotary base for the adapter key term; 0 disables it.
 *   dtype         LRA_BF16 (split-K kernel on MFMA, fp32 accumulate) or
 *                 LRA_F32 (fp32 throughout). With LRA_BF16 the adapter part
 *                 of each score is taken in f16: the rebuilt adapter key
 *                 rope(L_k B_k) is formed in fp32, converted to f16 and
 *                 rotated in f16, and q is converted to f16 for that product;
 *                 |q| and the rebuilt adapter-key entries must stay below
 *                 65504 (the f16 range), else the output is undefined.
 *   workspace     at least lora_attn_decode_workspace_size(...) bytes of
 *                 device memory, 16-byte aligned; it holds fp32 split-K
 *                 partial states (per split and query row: max, sum and the
 *                 value accumulator with the adapter term already applied),
 *                 never a full-dimension adapter key or value. Its contents
 *                 on entry do not matter. Calls that overlap in time must use
 *                 different workspaces. May be NULL when the size is 0.
 *   A call with bf16 is one main kernel, plus a combine kernel when a context
 *   is split; with f32 it is one kernel.
 * ---------------------------------------------------------------------- */
size_t lora_attn_decode_workspace_size(int32_t S, int32_t num_groups, int32_t Hq, int32_t Hkv, int32_t d,
                                       int32_t max_rank, int32_t max_context_len, int32_t dtype);

int lora_attn_decode(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                     int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                     const int32_t* group_offsets, int32_t num_groups, const int32_t* agent_ids,
                     const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools, const void* const* b_k,
                     const void* const* b_v, const int32_t* ranks, int32_t max_rank, int32_t S, int32_t N_agents,
                     int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size, float sm_scale, float rope_theta,
                     int32_t dtype, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention without a workspace, for callers that cannot allocate
 * device memory around the call (code being captured into a HIP graph,
 * tight serving loops, harnesses that forbid allocation). Arguments, result
 * and kernels are those of lora_attn_decode, less the workspace: the split
 * records go to a fixed device array of 16 MiB that the library holds on
 * each GPU it runs on until the process ends (its address is looked up once
 * per device, on the first call for that device). No call allocates or
 * frees anything.
 *   A call whose records need more than 16 MiB
 *   (lora_attn_decode_workspace_size) returns LRA_ERR_UNSUPPORTED before any
 *   HIP call. Every record a call reads is written by the same call, so the
 *   array needs no clearing; it keeps the last call's contents. All calls on
 *   one GPU share the array: calls that overlap in time on one GPU race and
 *   give undefined results (serialise them, e.g. on one stream).
 * ---------------------------------------------------------------------- */
int lora_attn_decode_noalloc(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                             const int32_t* group_offsets, int32_t num_groups, const int32_t* agent_ids,
                             const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools,
                             const void* const* b_k, const void* const* b_v, const int32_t* ranks, int32_t max_rank,
                             int32_t S, int32_t N_agents, int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                             float sm_scale, float rope_theta, int32_t dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Prefill attention: a chunk of q_len_s = cu_q_lens[s+1] - cu_q_lens[s]
 * new tokens per sequence, already written to the caches, attends causally:
 * query i of sequence s sits at position T_s - q_len_s + i and sees keys
 * 0..that position. PReCache runs adapted prefill over each agent's new
 * segment after a shared context (Figure 1 caption).
 *
 *   q, out        [cu_q_lens[S], Hq, d]; cu_q_lens int32 [S+1], q_len_s <= T_s.
 *   max_q_len     (host) >= every q_len_s.
 *   Everything else as for decode (no grouping; agent id -1, adapter_start
 *   and NULL b_k / b_v as there: without a key adapter the key tiles are the
 *   base keys as stored, without a value adapter the value tiles are the base
 *   values; key tiles wholly before the activation point read no low-rank
 *   rows). With a value adapter the values are kept in rank space (P L_v,
 *   then B_v once per row), except at rank 64 with both adapters, where each
 *   64-key tile's values are rebuilt as V + L_v B_v in LDS and rounded once
 *   to bf16, like the keys; either way nothing of full dimension is written
 *   to device memory.
 *   dtype: LRA_BF16, d = 128.
 *   workspace     lora_attn_prefill_workspace_size(...) bytes (may be 0,
 *                 then workspace may be NULL).
 * ---------------------------------------------------------------------- */
size_t lora_attn_prefill_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t max_rank,
                                        int32_t max_q_len, int32_t max_context_len, int32_t dtype);

int lora_attn_prefill(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                      int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len,
                      const int32_t* cu_q_lens, int32_t max_q_len, const int32_t* agent_ids,
                      const int32_t* adapter_start, const void* const* l_k_pools, const void* const* l_v_pools, const void* const* b_k,
                      const void* const* b_v, const int32_t* ranks, int32_t max_rank, int32_t S, int32_t N_agents,
                      int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size, float sm_scale, float rope_theta,
                      int32_t dtype, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode rows and prefill chunks in one call (a serving step that mixes
 * decoding sequences with prefill chunks: PReCache, Figure 1 caption, an
 * agent's new segment prefilled while other agents decode; LRAgent: Efficient
 * KV Cache Sharing for Multi-LoRA LLM Agents, abstract, concurrent agents on
 * one shared base). Sequences 0 .. S_dec - 1 decode (one query each), the
 * rest are prefill chunks. Each row's result is bit-identical to what
 * lora_attn_decode (for the first S_dec sequences) and lora_attn_prefill (for
 * the rest) would write.
 *
 *   q, out        [cu_q_lens[S], Hq, d]: decode sequence s < S_dec owns row s,
 *                 prefill sequence s its rows cu_q_lens[s] .. cu_q_lens[s+1]-1.
 *   cu_q_lens     int32 [S+1] with cu_q_lens[s] = s for s <= S_dec (device
 *                 memory: trusted by liblra.so, checked by liblra_debug.so);
 *                 may be NULL when S == S_dec.
 *   max_q_len     (host) >= every prefill q_len_s (>= 1).
 *   group_offsets int32 [num_groups+1] over the decode sequences only
 *                 (0 .. S_dec), as for decode; NULL: each decode sequence its
 *                 own group (num_groups ignored).
 *   block_tables, context_lens, agent_ids, adapter_start: one entry (row) per
 *                 sequence, decode sequences first.
 *   Everything else as for decode and prefill. dtype: LRA_BF16, d = 128.
 *   workspace     lora_attn_varlen_workspace_size(...) bytes (the decode
 *                 part's split records), as for decode.
 *   A call runs the prefill kernel for the chunks, then the decode kernel
 *   (and its combine kernel when a decode context is split) on `stream`.
 * ---------------------------------------------------------------------- */
size_t lora_attn_varlen_workspace_size(int32_t S, int32_t S_dec, int32_t num_groups, int32_t Hq, int32_t Hkv, int32_t d,
                                       int32_t max_rank, int32_t max_context_len, int32_t dtype);

int lora_attn_varlen(const void* q, const void* k_base, const void* v_base, const int32_t* block_tables,
                     int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len, const int32_t* cu_q_lens,
                     int32_t max_q_len, int32_t S, int32_t S_dec, const int32_t* group_offsets, int32_t num_groups,
                     const int32_t* agent_ids, const int32_t* adapter_start, const void* const* l_k_pools,
                     const void* const* l_v_pools, const void* const* b_k, const void* const* b_v, const int32_t* ranks,
                     int32_t max_rank, int32_t N_agents, int32_t Hq, int32_t Hkv, int32_t d, int32_t block_size,
                     float sm_scale, float rope_theta, int32_t dtype, void* out, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LRA_H */
