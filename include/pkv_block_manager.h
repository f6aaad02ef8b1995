/*
 * pkv_block_manager.h -- host-side block manager of libpagedkv.so: the
 * physical block pool, per-sequence block tables and the prefix cache that
 * feed the paged kernels (include/pagedkv.h).  Plain host memory only; no
 * GPU call is made.
 *
 * Pages cited (by title and section):
 *   [A] "KV-Cache Engineering: Paged Attention, Prefix Cache,
 *        Disaggregation (2026)" -- "How does prefix caching work",
 *        "What is cross-layer KV sharing".
 *   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
 *        Attention Variants, and the Bandwidth Wall" -- "PagedAttention",
 *        "Continuous Batching", "Prefix Caching".
 *   [C] "KV-Cache Engineering: The Memory Wall of LLM Serving" -- "When
 *        the cache fills".
 *
 * Model ([B] "PagedAttention"): num_blocks physical blocks of block_size
 * token slots; a sequence's table maps its logical block j to a physical
 * block; only the last block of a sequence is partly filled; any free block
 * serves any sequence; a retiring sequence returns its blocks.
 *
 * Prefix cache ([A] "How does prefix caching work", [B] "How vLLM
 * implements automatic prefix caching"): every FULL block is keyed by a
 * cumulative 128-bit hash of the token ids from the start of the sequence
 * to the end of that block (seeded by hash_namespace); a new sequence walks
 * its prompt block by block and maps each block whose key is cached into
 * its table, stopping at the first miss.  Cached blocks that no sequence
 * uses stay cached and are evicted least-recently-released first ([C]
 * "When the cache fills") only when no block is free.  The hash is not
 * collision-resistant against an adversary (two different prefixes with
 * equal 128-bit keys would share KV).
 *
 * Layer groups ([A] "What is cross-layer KV sharing": the key is taken per
 * layer group, not per layer): one manager's tables serve every layer
 * group of a model (each group has its own pool, indexed by the same
 * physical block ids), so each block has one key for all groups;
 * hash_namespace separates caches whose KV differs for equal tokens.
 *
 * Policy (the pages leave these open): a new block is the lowest-numbered
 * free block; a sequence's blocks are released last logical block first; a
 * prompt reuses only full blocks inside its first n - 1 tokens (the last
 * token is always computed); a block is keyed when it becomes full unless
 * its key is already held by another block; appending to a partly filled
 * block that forked sequences share first copies it (copy-on-write: the
 * caller copies the block's first valid_tokens slots, e.g. with
 * paged_kv_copy_blocks, before writing).  An operation that cannot get its
 * blocks returns PKV_ENOSPACE and changes nothing.
 *
 * KV writes: after pkv_bm_add the caller computes and writes the KV of
 * tokens [cached_tokens, n); after pkv_bm_append, of the appended tokens.
 * A block is keyed as soon as it is full in a table, so the caller must
 * write its KV before any other sequence's attention reads it (within a
 * step: writes before attention on one stream).
 *
 * Thread safety: every call locks the manager; calls on different managers
 * are independent.  Errors: PKV_EINVAL (null pointer, unknown or duplicate
 * sequence id, n < 1, bad sizes), PKV_ENOSPACE, PKV_ENOMEM.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks >= 1 blocks of block_size >= 1 slots, or NULL. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int64_t hash_namespace);
void pkv_bm_destroy(pkv_block_manager* bm);

/* New sequence `seq` with prompt tokens[0, n), n >= 1.  Writes to
 * *cached_tokens the number of leading tokens whose KV is already cached
 * (a multiple of block_size, at most n - 1). */
int pkv_bm_add(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n,
               int32_t* cached_tokens);

/* Extends `seq` by tokens[0, n) (one decode step, or a chunk), n >= 0. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n);

/* One call per step: appends tokens[token_start[i], token_start[i+1]) to
 * seqs[i] for i = 0, 1, ... in order, as pkv_bm_append would, stopping at
 * the first sequence that fails.  Returns the number of sequences extended
 * (n_seqs on full success); if the first one fails, its negative status. */
int32_t pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seqs, int32_t n_seqs,
                            const int32_t* token_start, const int32_t* tokens);

/* `child` starts as a copy of `parent` sharing all of its blocks. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Retires `seq`: its blocks go back to the free list, or, if keyed, to
 * the end of the eviction (LRU) list. */
int pkv_bm_release(pkv_block_manager* bm, int64_t seq);

/* Copy-on-write copies made since the last call, oldest first, as
 * (source block, destination block, valid tokens) triples in out[3 * i];
 * at most max_copies are returned and removed; returns their number. */
int32_t pkv_bm_take_copies(pkv_block_manager* bm, int32_t* out, int32_t max_copies);

/* Tokens of `seq` (>= 0), or a negative status. */
int32_t pkv_bm_context_len(pkv_block_manager* bm, int64_t seq);

/* Writes the table of `seq` into row[0, width), padded with -1; returns
 * its number of blocks, PKV_EINVAL if width is too small. */
int32_t pkv_bm_table(pkv_block_manager* bm, int64_t seq, int32_t* row, int32_t width);

/* One step's kernel inputs for n_seqs sequences in the given order:
 * block_tables [n_seqs, width] (padded with -1) and context_lens [n_seqs]
 * (host buffers; the caller copies them to the device). */
int pkv_bm_export(pkv_block_manager* bm, const int64_t* seqs, int32_t n_seqs,
                  int32_t* block_tables, int32_t width, int32_t* context_lens);

/* Counters into out[0, n) (n <= 8): free blocks, evictable cached blocks,
 * cached keys, live sequences, prompt blocks found in the cache, prompt
 * blocks looked up, evictions, copy-on-write copies. */
int pkv_bm_stats(pkv_block_manager* bm, int64_t* out, int32_t n);

/* Reference count of a block (number of tables naming it), or PKV_EINVAL. */
int32_t pkv_bm_ref(pkv_block_manager* bm, int32_t block);

/* The evictable blocks, least recently released first (at most max);
 * returns their total number. */
int32_t pkv_bm_lru(pkv_block_manager* bm, int32_t* out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
