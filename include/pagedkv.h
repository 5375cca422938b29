/*
 * pagedkv — paged KV cache for generation-phase attention on AMD Instinct
 * MI355X (gfx950). C ABI of libpagedkv.so.
 *
 * The method (sources: «The KV Cache and PagedAttention», world.lapla.si/en/kvcache,
 * and «KV cache», tellworld.net/learn/kv-cache):
 *  - each text's keys and values are cut into blocks of `block_size` token
 *    places; the text sees its blocks as consecutive logical blocks while
 *    the physical blocks can be anywhere ("Like Pages of Memory");
 *  - a per-text block table maps logical to physical blocks and records how
 *    many places of each are filled; a new block is taken only when the
 *    previous ones are full ("The Block Table");
 *  - blocks can be shared with reference counts and are copied before a
 *    sharer writes into them ("Shared, Copied on Write");
 *  - every generation step writes the new token's key and value and lets
 *    its query attend over the whole cache ("One Token at a Time"; «KV cache»
 *    "How it works").
 *
 * Conventions
 *  - Every call returns int status: PA_OK or a negative PA_E* code; nothing
 *    aborts or throws across the ABI. pa_last_error() gives a message for the
 *    last failing call on the calling thread.
 *  - Host allocator functions (pa_alloc_*, pa_seq_*, pa_step_append,
 *    pa_export_tables, ...) touch only host memory; all their pointers are
 *    host pointers. One pa_alloc must not be used from two threads at once.
 *  - Device functions (pa_kv_write, pa_copy_blocks, pa_decode_*) take device
 *    pointers the caller owns, enqueue work on `stream` (a hipStream_t; NULL
 *    is the null stream) and return without waiting. Host-side checks cover
 *    null pointers, sizes, dtype and 16-byte alignment; indices stored in
 *    device memory are bounds-guarded inside the kernels as stated per call, and the
 *    promises the calls take on trust can be re-checked (pa_set_debug_checks).
 *  - Layouts (row-major, contiguous):
 *      k_cache, v_cache  [num_blocks][num_kv_heads][block_size][head_dim]
 *      q, out            [num_seqs][num_heads][head_dim]
 *      k_new, v_new      [num_tokens][num_kv_heads][head_dim]
 *      block_tables      int32 [num_seqs][max_blocks_per_seq], unused entries -1
 *      context_lens      int32 [num_seqs], tokens attended, new token included
 *      slots             int64 [num_tokens], slot = physical_block * block_size + place
 *      pairs             int32 [num_pairs][2] = (source block, destination block)
 *    The K and V pools share physical block ids: one block holds the keys and
 *    the values of the same tokens.
 *  - Supported: dtype PA_F32 / PA_F16 / PA_BF16 (K, V, q and out share it),
 *    head_dim 64 or 128, block_size 4, 8, 16 or 32,
 *    num_heads a multiple of num_kv_heads (heads sharing key/value sets,
 *    "What Came After").
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_EINVAL = -1,        /* bad argument: null, out of range, misaligned */
  PA_ENOBLOCKS = -2,     /* not enough free blocks; nothing was changed */
  PA_ENOSEQ = -3,        /* unknown or released sequence id */
  PA_EHIP = -4,          /* a HIP runtime call failed (message has the HIP error) */
  PA_EUNSUPPORTED = -5   /* valid but not supported (dtype, head_dim, block_size) */
};

/* Element formats. PA_FP8_E4M3 (OCP FP8 E4M3, one byte a number) is for key/value pools
 * only: see pa_kv_write_fp8 and pa_decode_attention_fp8. */
enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 };

/* Message for the last failing call on this thread ("" if none). Owned by the library. */
const char* pa_last_error(void);
/* Library ABI version (major*100 + minor). */
int pa_version(void);

/* ---------------------------------------------------------------------------
 * Host block allocator ("The Block Table", "Shared, Copied on Write",
 * "When Memory Runs Out").
 *
 * Policy (fixed so that block tables are reproducible):
 *  - The free list is a stack. With free_order given, free_order[0] is handed
 *    out first; without it, block 0 first. Blocks released by pa_seq_free are
 *    pushed in logical order, so the released text's last block comes next.
 *  - Sequence ids count up from 0 and are never reused.
 *  - pa_seq_append gives a text a new block only when its last block is full.
 *    If its last block is partly filled and shared (count > 1), the block is
 *    first replaced by a fresh copy target: the caller must copy source ->
 *    destination (pa_copy_blocks) before writing any new token. The original's
 *    count drops by one, so the last remaining holder writes in place. A
 *    shared block that is full is never copied.
 *  - All-or-nothing: if the free list cannot supply every block an append
 *    needs, PA_ENOBLOCKS is returned and nothing changes.
 * ------------------------------------------------------------------------- */
typedef struct pa_alloc pa_alloc;

/* num_blocks >= 1, block_size >= 1; free_order: NULL or a permutation of 0..num_blocks-1. */
int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pa_alloc** out);
void pa_alloc_destroy(pa_alloc* a);

/* New empty text. */
int pa_seq_add(pa_alloc* a, int32_t* seq_out);
/* New text sharing every block of `parent` (each block's count + 1) — parallel sampling. */
int pa_seq_fork(pa_alloc* a, int32_t parent, int32_t* child_out);
/* Slots for n_tokens new tokens of `seq` (n_tokens >= 0), in token order.
 * *cow_src / *cow_dst: the block to copy and its copy, or -1 / -1. */
int pa_seq_append(pa_alloc* a, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                  int32_t* cow_src, int32_t* cow_dst);
/* One generation step for n texts, in order: one token each (pa_seq_append(seqs[i], 1)).
 * slots_out[n]; pairs_out[n][2] receives the copy pairs in order, *num_pairs_out their count.
 * On PA_ENOBLOCKS the first *done_out texts have been appended (their slots and pairs are
 * valid) and text seqs[*done_out] and later are unchanged. */
int pa_step_append(pa_alloc* a, const int32_t* seqs, int32_t n, int64_t* slots_out,
                   int32_t* pairs_out, int32_t* num_pairs_out, int32_t* done_out);
/* Release a text: each of its blocks' counts - 1; blocks reaching 0 return to the free list. */
int pa_seq_free(pa_alloc* a, int32_t seq);
/* Tokens held and blocks used by `seq`. */
int pa_seq_info(const pa_alloc* a, int32_t seq, int32_t* ctx_len, int32_t* n_blocks);
/* Block-table entries of `seq`: physical block and filled places per logical block
 * (cap = capacity of both arrays; PA_EINVAL if too small). */
int pa_seq_block_table(const pa_alloc* a, int32_t seq, int32_t* phys_out, int32_t* filled_out,
                       int32_t cap);
/* Dense tables for a batch: tables_out[n][max_blocks_per_seq] (unused entries -1) and
 * ctx_lens_out[n]. PA_EINVAL if a text has more than max_blocks_per_seq blocks. */
int pa_export_tables(const pa_alloc* a, const int32_t* seqs, int32_t n,
                     int32_t max_blocks_per_seq, int32_t* tables_out, int32_t* ctx_lens_out);
/* Reference count of a physical block (0 = free). */
int pa_block_ref(const pa_alloc* a, int32_t block, int32_t* ref_out);
int pa_num_free(const pa_alloc* a, int32_t* n_out);
/* Blocks in use and filled places over them (each physical block counted once):
 * filled / (used * block_size) is the share of the cache holding tokens ("What It Does"). */
int pa_alloc_stats(const pa_alloc* a, int64_t* used_blocks, int64_t* filled_slots);

/* Share groups of a batch for pa_decode_attention_prefix / _prefix2, read off the block
 * tables ("Shared, Copied on Write": texts forked from one another hold their common
 * blocks in common, with counts), so that the groups' promise (members' tables begin with
 * the same blocks) holds by construction.
 * pa_share_groups: maximal runs of consecutive batch texts seqs[i], seqs[i+1], ... (at most
 * max_members, >= 2) that all hold the run's first text's first block; each run of two or
 * more texts is a group: first_out = its first batch index, count_out = its texts,
 * prefix_out = the leading blocks all its members hold in common, times block_size (the
 * decode clamps that to each member's context less one token). Texts in no run are in no
 * group. Outputs [cap]; *num_groups_out groups (PA_EINVAL if more than cap).
 * pa_share_groups_inner: inside each given group (first, count, prefix as above), maximal
 * runs of at most inner_members (>= 2) consecutive members that hold more leading blocks in
 * common than prefix / block_size: the inner level of pa_decode_attention_prefix2 (a pair
 * of beams also shares the tokens written since the two split).
 * Swapped-out texts: PA_EINVAL; unknown ids: PA_ENOSEQ. */
int pa_share_groups(const pa_alloc* a, const int32_t* seqs, int32_t n, int32_t max_members,
                    int32_t cap, int32_t* first_out, int32_t* count_out, int32_t* prefix_out,
                    int32_t* num_groups_out);
int pa_share_groups_inner(const pa_alloc* a, const int32_t* seqs, int32_t n, int32_t num_groups,
                          const int32_t* group_first, const int32_t* group_count,
                          const int32_t* group_prefix, int32_t inner_members, int32_t cap,
                          int32_t* first_out, int32_t* count_out, int32_t* prefix_out,
                          int32_t* num_inner_out);

/* ---------------------------------------------------------------------------
 * Swapping to host memory («The KV Cache and PagedAttention», "When Memory Runs Out":
 * when blocks run short, a text gives up all of its blocks at once; one answer is to
 * move them to the CPU's memory and back when the text's turn comes).
 *
 * The allocator keeps a second pool of num_host_blocks blocks in host memory, a stack
 * like the device free list (free_order[0] handed out first, else block 0). Swapping
 * a list of texts moves every block they hold: each distinct block once (texts in list
 * order, logical blocks in order, first occurrence), so blocks the listed texts share
 * stay shared on the other side, with a count of the listed texts holding them. Blocks
 * also held by texts not listed are copied and stay where they are for those texts.
 * The caller moves the bytes with pa_swap_blocks, out before the device blocks are
 * reused, in before the texts are next attended. A swapped-out text cannot be appended
 * to, forked, exported or registered (PA_EINVAL); pa_seq_free releases its host blocks;
 * pa_seq_info and pa_seq_block_table report its host blocks.
 * ------------------------------------------------------------------------- */
/* Set up the host pool once (PA_EINVAL if already set up). free_order: NULL or a
 * permutation of 0..num_host_blocks-1. */
int pa_alloc_host_pool(pa_alloc* a, int32_t num_host_blocks, const int32_t* free_order);
/* Move texts seqs[0..n-1] (live, resident, each listed once) to host blocks. pairs_out
 * [cap][2] receives (device block, host block) per distinct block; *num_pairs_out their
 * number. Device blocks no text holds any more return to the free list in that order
 * (as pa_seq_free releases them). All-or-nothing: PA_ENOBLOCKS if the host pool has too
 * few free blocks, PA_EINVAL if cap is too small; nothing changes then. */
int pa_swap_out(pa_alloc* a, const int32_t* seqs, int32_t n, int32_t* pairs_out, int32_t cap,
                int32_t* num_pairs_out);
/* Bring swapped-out texts back: pairs_out receives (host block, device block) per
 * distinct host block, device blocks taken from the free list's top in that order;
 * host blocks no text holds any more return to the host stack in that order.
 * All-or-nothing as pa_swap_out (PA_ENOBLOCKS: too few free device blocks). */
int pa_swap_in(pa_alloc* a, const int32_t* seqs, int32_t n, int32_t* pairs_out, int32_t cap,
               int32_t* num_pairs_out);
/* 1 if `seq` is swapped out, else 0. */
int pa_seq_swapped(const pa_alloc* a, int32_t seq, int32_t* swapped_out);
/* Count of a host block (0 = free), and the free host blocks. */
int pa_host_block_ref(const pa_alloc* a, int32_t block, int32_t* ref_out);
int pa_host_num_free(const pa_alloc* a, int32_t* n_out);

/* ---------------------------------------------------------------------------
 * Debug re-checks of what the device calls take on trust (on the host, before launch):
 *  - pa_kv_write, pa_kv_write_fp8: the slots inside the pool are distinct;
 *  - pa_decode_attention_write, pa_decode_attention_prefix2_write, and
 *    pa_decode_attention_prefix2_run with new rows: also, each text's slot
 *    is the place of its last attended position in its table;
 *  - pa_copy_blocks: destinations distinct, no block both a source and a destination;
 *  - pa_decode_attention_prefix / _prefix2 / pa_decode_prefix2_plan: no text in two groups
 *    of one level, and every member's table holds its group's first member's blocks over
 *    the blocks the level reads once for the group (with the decode's own clamps).
 * A failed check returns PA_EINVAL naming the offender, and nothing is launched. Each check
 * copies the device arrays it needs to the host and waits for `stream`: for testing, not
 * for the timed path. Off by default; on when PA_DEBUG_CHECKS is set to a value other than
 * "0" in the environment when first consulted, or after pa_set_debug_checks(1).
 * pa_debug_checks() returns 1 when on. */
int pa_set_debug_checks(int32_t on);
int pa_debug_checks(void);

/* ---------------------------------------------------------------------------
 * Device cache writes.
 * ------------------------------------------------------------------------- */

/* Write each new token's key and value into its slot ("One Token at a Time"):
 *   k_cache[slot/B][h][slot%B][:] = k_new[i][h][:] for every kv head h; same for V.
 * Bit-exact copy. Slots must be distinct. A slot outside [0, num_blocks*block_size)
 * is skipped (nothing written for that token). num_tokens == 0 is a no-op. */
int pa_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                const int64_t* slots, int32_t num_tokens, int32_t num_blocks,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                void* stream);

/* Copy whole blocks, keys and values, for copy-on-write ("Shared, Copied on Write"):
 *   k_cache[dst] = k_cache[src], v_cache[dst] = v_cache[src] for each pair.
 * Pairs are copied concurrently: destinations must be distinct and no block may be
 * both a source and a destination in one call (the allocator's pairs satisfy this).
 * A pair with an index outside [0, num_blocks) is skipped. dtype may be PA_FP8_E4M3. */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t dtype, void* stream);

/* Move whole blocks between two pools of the same shape, for swapping ("When Memory Runs
 * Out"): for each pair (src, dst) in order, block src of src_k / src_v is copied to block
 * dst of dst_k / dst_v, bit for bit. One side is normally pinned host memory (hipHostMalloc;
 * torch pin_memory), the other device memory; the kernel reads and writes host memory
 * directly (one launch for all pairs). pairs: int32 [num_pairs][2] in device memory or
 * pinned host memory. Every pointer is checked with hipPointerGetAttributes: device memory
 * or pinned host memory, else PA_EINVAL (pageable host memory is refused before anything
 * is launched). Pools: [num_src_blocks] / [num_dst_blocks] x [num_kv_heads][block_size]
 * [head_dim], 16-byte aligned; the pools must not overlap. A pair with an index outside its
 * pool is skipped. dtype may be PA_FP8_E4M3. Stream-ordered; host memory must stay
 * allocated until the copy has finished. */
int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int32_t* pairs, int32_t num_pairs, int32_t num_src_blocks,
                   int32_t num_dst_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t dtype, void* stream);

/* Like pa_kv_write into PA_FP8_E4M3 pools ("What Came After": the cache kept in 8-bit
 * floating point, one byte a number). k_new / v_new hold src_dtype values (PA_F32,
 * PA_F16 or PA_BF16); each is stored as the E4M3 code of fp32(x) * fp32(1 / scale)
 * (k_scale for keys, v_scale for values): round to nearest even, magnitudes beyond 448
 * saturate to 448, NaN stays NaN. Scales must be finite and > 0. */
int pa_kv_write_fp8(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int64_t* slots, int32_t num_tokens, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t src_dtype, float k_scale, float v_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Decode attention ("One Token at a Time"; «KV cache» "How it works";
 * "The Block Table": the kernel follows the table to each block).
 *
 *   out[s][h][:] = sum_t p_t * V_s[t],  p = softmax_t(scale * <q[s][h], K_s[t]>),
 *   t over the context_lens[s] tokens of text s in logical order, K_s[t] / V_s[t]
 *   read from physical block block_tables[s][t / block_size], place t % block_size,
 *   key/value head h / (num_heads / num_kv_heads).
 *
 * The work over all (text, head, 16-token chunk) units is cut into equal
 * contiguous segments, one per wavefront; a text's chunks can span several
 * segments, whose partial results (running max, sum, weighted values; fp32) are
 * merged by a second kernel in segment order. Accumulation is fp32; out is
 * rounded to nearest even. The result depends only on logical positions, never on
 * block placement.
 *
 * partition_tokens: 0 = 4 segments per compute unit (recommended); else a multiple
 *   of 16 giving the segment length in tokens.
 * max_context_len: upper bound of context_lens (sizes the segment grid).
 * context_lens[s] == 0 gives zeros. A table entry outside [0, num_blocks) for an
 * attended token, or context_lens[s] > max_blocks_per_seq * block_size, makes
 * out[s][:][:] NaN (nothing outside the pools is read).
 * workspace: device memory of at least pa_decode_workspace_bytes(...) bytes for the
 * same num_seqs, num_heads, head_dim, max_context_len, partition_tokens on the
 * current device; its contents need no initialisation. Calls sharing a workspace
 * must be ordered on one stream. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens);
/* Zero `workspace_bytes` bytes of a decode workspace on `stream` (a fill kernel, not a
 * memset, so it may be recorded into a HIP graph). Optional: for byte-reproducible
 * workspace contents. */
int pa_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);
int pa_decode_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t max_context_len,
                        int32_t partition_tokens, float scale, int32_t dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode_attention without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The workspace is the library's own: a device array of
 * pa_decode_noalloc_max_bytes() = 16 MiB, one copy per GPU (devices 0..63), set up on the
 * first call on each device and held until the process ends. This call allocates nothing.
 * A launch whose workspace (pa_decode_workspace_bytes for the same arguments) would exceed
 * it is refused with PA_EINVAL before anything is launched: with partition_tokens 0 a
 * head_dim-128 launch needs 8.7 MB plus 8 bytes per text on 256 compute units. Every call
 * on one GPU uses the same array: calls that may overlap on one GPU (two streams, two
 * threads) race and give wrong results; order them on one stream. The array needs no
 * clearing (each launch writes what it reads). Otherwise as pa_decode_attention. */
size_t pa_decode_noalloc_max_bytes(void);
int pa_decode_attention_noalloc(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                int32_t partition_tokens, float scale, int32_t dtype,
                                void* stream);

/* Decode attention over PA_FP8_E4M3 pools: every stored key is decode(code) * k_scale,
 * every value decode(code) * v_scale; q and out are q_dtype (PA_F16 or PA_BF16).
 * Otherwise as pa_decode_attention (same workspace sizing). */
int pa_decode_attention_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            int32_t partition_tokens, float scale, float k_scale, float v_scale,
                            int32_t q_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Decode attention with the step's new-token write fused in (one launch instead of
 * pa_kv_write then pa_decode_attention; «KV cache» "How it works": the new position's
 * key and value join the cache and are attended in the same step).
 *
 * Result, bit for bit, that of
 *   pa_kv_write(k_cache, v_cache, k_new, v_new, slots', num_seqs, ...);
 *   pa_decode_attention(out, q, k_cache, v_cache, ...);
 * with slots'[s] = slots[s] for texts with context_lens[s] >= 1 and -1 (skipped) for the
 * others, provided slots[s] is the place of position context_lens[s] - 1 of text s in
 * its block table (what pa_step_append hands out) and no text of the batch attends
 * another text's new place (copy-on-write guarantees it). The last position's key and
 * value are read from k_new / v_new; one wave per (text, key/value head) stores them
 * into the pools during the launch, for later steps. Slots outside
 * [0, num_blocks * block_size) are skipped.
 *
 * k_new, v_new: [num_seqs][num_kv_heads][head_dim] in dtype, 16-byte aligned; slots:
 * int64 [num_seqs]. dtype PA_F32, PA_F16 or PA_BF16 (E4M3 pools: pa_kv_write_fp8, then
 * pa_decode_attention_fp8). Everything else, the workspace included, as
 * pa_decode_attention. */
int pa_decode_attention_write(void* out, const void* q, void* k_cache, void* v_cache,
                              const void* k_new, const void* v_new, const int64_t* slots,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              int32_t partition_tokens, float scale, int32_t dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Decode over shared prompt blocks. Texts forked from one prompt (parallel sampling, beam
 * search: "Shared, Copied on Write", the samples of one request hold the
 * prompt's blocks in common) read those blocks once per group instead of once per text.
 * Same result as pa_decode_attention (up to rounding: two softmax partials merged).
 *   Group g: texts group_first[g] .. group_first[g] + group_count[g] - 1 (device int32
 *   arrays [num_groups], like group_prefix), whose tables begin with the same
 *   group_prefix[g] / block_size blocks (the caller's promise; the group's first member's
 *   table row is read for them). group_prefix[g] is taken at most max_prefix_len and
 *   every member's context length - 1 (each member keeps its newest token to itself),
 *   rounded down to a block. At most 8 / (num_heads / num_kv_heads) members per group
 *   (more are left out of the group; larger sharing sets: several groups over the same
 *   blocks); group_first clamped into the batch. Groups must not overlap (a text in two
 *   groups: result unspecified). Texts in no group decode as usual.
 * Three passes on `stream`: group set-up, the groups' shared blocks (each key/value row
 * read once for all members: the members' heads as one key/value head's 8 query heads),
 * each text's own blocks with the shared part's softmax state folded in. No new-token
 * write here (pa_kv_write first). dtype PA_F32, PA_F16 or PA_BF16; num_heads /
 * num_kv_heads <= 8 (else PA_EUNSUPPORTED). num_groups 0: pa_decode_attention.
 * workspace: pa_decode_prefix_workspace_bytes(...) bytes, 16-byte aligned, no
 * initialization needed; overlapping calls on one workspace race. */
size_t pa_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len,
                                        int32_t num_groups, int32_t max_prefix_len,
                                        int32_t dtype);
int pa_decode_attention_prefix(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int32_t num_groups,
                               const int32_t* group_first, const int32_t* group_count,
                               const int32_t* group_prefix, int32_t max_prefix_len, float scale,
                               int32_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Decode over shared blocks at two nested levels, for sharing trees two deep (beam search:
 * a request's samples share its prompt, and a pair of beams also shares the tokens written
 * since they split; "Shared, Copied on Write"). Each shared block is read once for all the
 * texts that hold it. The outer groups are pa_decode_attention_prefix's groups; an inner
 * group's members share the blocks from where their outer group's shared part ends up to
 * inner_prefix[g] (an inner group keeps its members up to the first whose outer shared
 * part differs from its first member's: members of different outer groups, or of none,
 * are not grouped together)
 * (clamped as for the outer level: at most max_inner_prefix_len, every member's context
 * less one token, a block multiple; an inner part no longer than the outer one is empty).
 * The inner groups' table entries are read from their first member's row. Same result as
 * pa_decode_attention up to rounding. At most 8 / (num_heads / num_kv_heads) members per
 * outer group and inner_members per inner group (more are left out of the group);
 * inner_members sets the width of the inner pass (its members' query heads per key/value
 * head, rounded up to 1, 2, 4 or 8: pairs of texts with one query head per key/value head
 * take the two-head vector kernel), PA_EUNSUPPORTED past 8. Passes on `stream`: the set-up
 * (pa_decode_prefix2_plan), then pa_decode_attention_prefix2_run: the outer groups' shared
 * blocks, the inner groups' shared blocks, one merge of both levels' partials into the
 * members' softmax states, every text's own blocks with both levels' states folded in (each
 * level's state used only where its start moved past the level before), and its merge. dtype, limits
 * and errors as pa_decode_attention_prefix; the group
 * arrays are device int32 [num_groups] and [num_inner_groups], both counts >= 1.
 * workspace: pa_decode_prefix2_workspace_bytes(...) bytes, 16-byte aligned, no
 * initialization needed. */
size_t pa_decode_prefix2_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t max_context_len,
                                         int32_t num_groups, int32_t max_prefix_len,
                                         int32_t num_inner_groups, int32_t max_inner_prefix_len,
                                         int32_t inner_members, int32_t dtype);
int pa_decode_attention_prefix2(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_context_len, int32_t num_groups,
                                const int32_t* group_first, const int32_t* group_count,
                                const int32_t* group_prefix, int32_t max_prefix_len,
                                int32_t num_inner_groups, const int32_t* inner_first,
                                const int32_t* inner_count, const int32_t* inner_prefix,
                                int32_t max_inner_prefix_len, int32_t inner_members,
                                float scale, int32_t dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* pa_decode_attention_prefix2 with the step's new-token write fused in ("Shared, Copied on
 * Write": forked texts append their own tokens; «KV cache» "How it works": the new
 * position's key and value join the cache and are attended in the same step).
 *
 * Result, bit for bit, that of
 *   pa_kv_write(k_cache, v_cache, k_new, v_new, slots', num_seqs, ...);
 *   pa_decode_attention_prefix2(out, q, k_cache, v_cache, ...);
 * with slots' and the conditions on slots as for pa_decode_attention_write (slots[s] the
 * place of position context_lens[s] - 1 of text s in its table; no text attends another's
 * new place). A text's newest token always lies in its own blocks (each level leaves every
 * member at least that token), so the texts' own pass reads it from k_new / v_new and
 * stores it into the pools (one wave per text and key/value head); the shared passes never
 * read it. Slots outside [0, num_blocks * block_size) are skipped. k_new, v_new:
 * [num_seqs][num_kv_heads][head_dim] in dtype, 16-byte aligned; slots: int64 [num_seqs].
 * Everything else, the workspace included, as pa_decode_attention_prefix2. */
int pa_decode_attention_prefix2_write(
    void* out, const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
    const int64_t* slots, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_groups, const int32_t* group_first, const int32_t* group_count,
    const int32_t* group_prefix, int32_t max_prefix_len, int32_t num_inner_groups,
    const int32_t* inner_first, const int32_t* inner_count, const int32_t* inner_prefix,
    int32_t max_inner_prefix_len, int32_t inner_members, float scale, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode_attention_prefix2 (and _write) in two parts, for a model whose layers all
 * attend with the same block tables, context lengths and groups in a decode step (the
 * tables map token positions to blocks for every layer: "The Block Table"): the set-up
 * once per step, then the passes once per layer.
 *
 * pa_decode_prefix2_plan writes into `workspace` what the tables, lengths and groups alone
 * decide: each group's shared length, table row and members, each text's start at both
 * levels and its outer group. One launch on `stream` (three past 2,048 texts or groups a
 * level); arguments, clamps and errors as pa_decode_attention_prefix2 (no q, pools or
 * output are read; the group arrays are read by this call only). With debug checks on it
 * re-checks the groups as pa_decode_attention_prefix2 does.
 *
 * pa_decode_attention_prefix2_run then runs that call's passes over the plan in
 * `workspace`, any number of times while the tables, lengths and groups stay as planned
 * (k_cache / v_cache and q may change: one call per layer). With k_new, v_new and slots
 * (all three, else all null) it also writes the new rows, as pa_decode_attention_prefix2_
 * write. The shapes, counts, max_prefix_len, max_inner_prefix_len, inner_members, dtype and
 * workspace_bytes must be those of the plan call. Result, bit for bit, that of
 * pa_decode_attention_prefix2 (_write) with the planned groups. The run overwrites the
 * workspace's partials and states but not the plan. A workspace holding no plan for these
 * arguments gives meaningless outputs without leaving the batch, the pools or the
 * workspace (the kernels clamp what they read there as they clamp the caller's indices).
 * A run must not overlap a plan or another run on the same workspace. */
int pa_decode_prefix2_plan(
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_groups,
    const int32_t* group_first, const int32_t* group_count, const int32_t* group_prefix,
    int32_t max_prefix_len, int32_t num_inner_groups, const int32_t* inner_first,
    const int32_t* inner_count, const int32_t* inner_prefix, int32_t max_inner_prefix_len,
    int32_t inner_members, int32_t dtype, void* workspace, size_t workspace_bytes,
    void* stream);
int pa_decode_attention_prefix2_run(
    void* out, const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
    const int64_t* slots, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_groups, int32_t max_prefix_len, int32_t num_inner_groups,
    int32_t max_inner_prefix_len, int32_t inner_members, float scale, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Prefix caching ("What Came After": every full block gets a hash of its tokens and
 * of everything before them; a request that begins the same way reuses the blocks,
 * which saves prompt-phase work only).
 *
 * Hash: 64-bit FNV-1a chained over blocks,
 *   h_j = FNV-1a(le64(h_{j-1}) || le32(tok[jB]) || ... || le32(tok[jB+B-1])),  h_{-1} = parent,
 * for the n_tokens / block_size full blocks (parent = 0 at a text's start).
 * Registered blocks: a hash maps to at most one block and a block carries at most
 * one hash. A registered block whose count drops to 0 stays registered and goes to
 * the bottom of the free stack (below every unregistered free block; of one text's
 * blocks the later ones above the earlier), so it is handed out last; handing it
 * out again drops its registration. Without registered blocks nothing changes in
 * the policy above.
 * ------------------------------------------------------------------------- */
int pa_hash_blocks(const int32_t* tokens, int32_t n_tokens, int32_t block_size,
                   uint64_t parent, uint64_t* hashes_out);
/* A new sequence starting on the registered blocks matching hashes[0], hashes[1], ...
 * up to the first miss (each count + 1; a free registered block is taken back out of
 * the free stack). *n_cached_out = blocks reused; the sequence holds
 * *n_cached_out * block_size tokens. To leave a prompt's last token to compute, pass
 * at most (prompt_len - 1) / block_size hashes. */
int pa_seq_add_cached(pa_alloc* a, const uint64_t* hashes, int32_t n_hashes, int32_t* seq_out,
                      int32_t* n_cached_out);
/* Register the sequence's first n blocks (all full, keys and values written) under
 * hashes[0..n-1]; a hash already registered or a block already registered is skipped.
 * PA_EINVAL (nothing changed) if n exceeds the sequence's blocks or one is not full. */
int pa_seq_cache_blocks(pa_alloc* a, int32_t seq, const uint64_t* hashes, int32_t n);
/* Registered blocks, and how many of them are free (count 0). */
int pa_cache_stats(const pa_alloc* a, int32_t* registered_out, int32_t* registered_free_out);

/* ---------------------------------------------------------------------------
 * Prompt phase ("One Token at a Time": a text's whole prompt at once; "What It
 * Does": each token attends every token before it; «KV cache» "How it works":
 * and its own). Causal attention of packed prompt queries over the paged cache.
 *
 *   rows q_start[s] .. q_start[s+1]-1 of q / out are text s's queries, its last
 *   n_s = q_start[s+1] - q_start[s] positions: row q_start[s] + i sits at position
 *   p = context_lens[s] - n_s + i and
 *   out[row][h][:] = sum_{t<=p} w_t * V_s[t],  w = softmax_{t<=p}(scale * <q[row][h], K_s[t]>),
 *   K_s / V_s read through the block table as in pa_decode_attention, key/value head
 *   h / (num_heads / num_kv_heads).
 * So the keys and values of the queries' own positions must already be in the cache
 * (write them with pa_kv_write first); positions before the queries are a cached
 * prefix (a reused prompt prefix, "What Came After"), possibly empty.
 *
 * q, out: [num_rows][num_heads][head_dim], dtype PA_F16 or PA_BF16 (pools the same);
 * q_start: int32 [num_seqs + 1], non-decreasing, 0 <= q_start[s] and
 * q_start[num_seqs] <= num_rows. Texts with q_start[s+1] <= q_start[s] are skipped;
 * rows of a text whose range leaves [0, num_rows) are not written.
 * max_q_len: the largest n_s (sizes the grid; larger n_s are still computed, slower).
 * Products run on the matrix cores with fp32 accumulation; the softmax weights are
 * rounded to the input format before they multiply the values; out is rounded to
 * nearest even. n_s > context_lens[s], context_lens[s] > max_blocks_per_seq *
 * block_size, or a table entry outside [0, num_blocks) for a needed position makes
 * that text's rows NaN (nothing outside the pools is read).
 * scale must be finite and > 0. Returns PA_EUNSUPPORTED for other dtypes, head_dim
 * other than 64/128, block_size other than 4/8/16/32. No workspace. */
int pa_prefill_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* q_start, int32_t num_seqs, int32_t num_rows,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_q_len, float scale, int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers (not part of the method): the achievable HBM read rate
 * and a copy of known size for calibrating memory counters.
 * ------------------------------------------------------------------------- */
/* Stream-read `bytes` (multiple of 16) from buf: each workgroup one contiguous range,
 * 16 non-temporal 16-byte loads in flight per lane; sink receives 4 bytes per workgroup
 * (size it with pa_probe_sink_bytes). waves_per_cu 0 = 4. */
size_t pa_probe_sink_bytes(int32_t waves_per_cu);
int pa_stream_read_probe(const void* buf, size_t bytes, void* sink, int32_t waves_per_cu,
                         void* stream);
/* Read the tiles tile_ids[0 .. n_ids) of tile_bytes each (2048, 4096, 8192 or 16384) from
 * buf, the access pattern of decode attention over randomly placed blocks: each of 4 waves
 * per CU reads a contiguous share of the list, 32 KiB in flight, non-temporal 16-byte
 * loads. Ids are clamped into [0, buf_bytes / tile_bytes). sink: pa_probe_sink_bytes(4). */
int pa_tile_read_probe(const void* buf, size_t buf_bytes, int32_t tile_bytes,
                       const int32_t* tile_ids, int64_t n_ids, void* sink, void* stream);
/* dst[0:bytes] = src[0:bytes] (bytes multiple of 16). */
int pa_copy_probe(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
