/*
 * rec.h — C ABI of librec, the gfx950 (MI355X) sparse embedding + DIN
 * attention forward.
 *
 * What is computed (pages; title and section):
 *   "MultiTowerDIN：当前现状分析" (MultiTowerDIN: current state)
 *     §2    id features arrive as jagged values + lengths (KeyedJaggedTensor)
 *     §3    each id feature owns a dense [num_buckets, 16] table; the row of a
 *           raw id is raw_id % num_buckets
 *     §4.1  click sequences are capped at 100 positions, real lengths ~3-5;
 *           padding them to 100 is the main waste — this library never pads
 *     §4.2  DIN attention: [q, s, q-s, q*s] -> attn MLP (256, 64) -> one
 *           score per position -> masked softmax -> weighted sum
 *     §4.4  shapes: pooled deep features, query [B,48], output [B,48]
 *   "MultiTowerDIN：集成 DynamicEmb" (integrating DynamicEmb)
 *     §1    a hash-table slot is key (8 B) + score (8 B) + digest (1 B) +
 *           16 fp32 values; §3.2 lookup is O(1) open addressing and an unseen
 *           id returns the constant 0 vector; §3.3 lookups stay fp32
 *   DLRM essay (wmrh.cn/news/12459) §3.2: EmbeddingBag sum pooling.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns and
 *     allocates every buffer, including workspaces; the library allocates
 *     nothing.  Its only state is a thread-local error message, a cache of
 *     each device's compute-unit count (read once per device, used to size
 *     persistent grids), and the thread-local timing events of
 *     rec_time_next_launch.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream).  Device buffers must stay alive until that work is done.
 *     Host structs and host arrays are read during the call only.
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns its error code, sets rec_last_error() and launches
 *     nothing.  Nothing throws across the ABI.  Zero-size work (B == 0,
 *     n == 0) returns REC_OK and launches nothing.
 *   - Preconditions the library does NOT check (device data): lengths >= 0;
 *     offsets consistent with lengths; sequence runs in bounds of their
 *     arrays; hash tables laid out as described below.  Violations are
 *     undefined behaviour.
 *   - Results are deterministic: the same inputs give bit-identical outputs run
 *     to run.  No floating-point sum depends on the order of atomics.  Three
 *     places use atomics, all on integers: rec_hash_insert and
 *     rec_hash_admit (64-bit compare-and-swap to claim free slots, counts and
 *     first positions; each documents what its placement may depend on), and
 *     the DIN plan (rec_din_plan, rec_din_attn_fwd, rec_sparse_din_fwd), which
 *     appends the samples without positions to a list with one atomic add per
 *     16 samples: the list's order may vary, but each of its samples only gets
 *     its zero output row, so no output depends on that order.
 */
#ifndef REC_H
#define REC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    REC_OK = 0,
    REC_EINVAL = -1,        /* a null required pointer, bad size/kind/dtype/alignment */
    REC_EUNSUPPORTED = -2,  /* valid but beyond this library's limits (see below) */
    REC_EHIP = -3,          /* a HIP runtime call failed; message holds hipGetErrorString */
    REC_EWORKSPACE = -4     /* workspace/plan missing or smaller than required */
} rec_status;

enum { REC_DIRECT = 0, REC_HASH = 1 };   /* rec_table.kind */
enum { REC_F32 = 0, REC_BF16 = 1, REC_BF16_PACKED = 2 };   /* rec_din_mlp.dtype */
enum { REC_SCORE_NONE = 0, REC_SCORE_STEP = 1, REC_SCORE_LFU = 2 };   /* rec_hash_insert */
enum { REC_TIME_DIN_ATTN = 0, REC_TIME_GATHER = 1, REC_TIME_SUMS = 2, REC_TIME_TOWERS = 3,
       REC_TIME_DLRM_INTERACT = 4, REC_TIME_DLRM_FWD = 5,
       REC_TIME_KINDS = 6 };                                        /* rec_time_next_launch */
enum { REC_POOL_SUM = 0, REC_POOL_MEAN = 1 };                    /* rec_dlrm_fwd bag modes */

#define REC_DIM 16                        /* embedding width of every table */
#define REC_EMPTY_KEY ((int64_t)-1)       /* empty hash slot; never a valid key */
#define REC_TOMBSTONE_KEY ((int64_t)-2)   /* slot of an evicted key (rec_hash_admit); never a valid key */
#define REC_MAX_TABLES 32                 /* tables per rec_embbag_fwd call */
#define REC_MAX_SEQ_LEN 1024              /* largest max_len for the DIN calls */
#define REC_MAX_B 16777215                /* largest batch for the DIN plan */
#define REC_DIN_PACKED_BYTES 106496       /* packed bf16 W1+W2 (rec_din_pack_mlp) */
#define REC_TOWER_PACKED_BYTES 614400     /* packed bf16 tower weights (rec_tower_pack_mlp) */
#define REC_NOALLOC_SCRATCH_BYTES 33554432 /* static scratch of rec_sparse_din_fwd_noalloc (32 MiB) */

/*
 * One embedding table (host struct; the arrays inside are device memory).
 *
 * kind == REC_DIRECT ("当前现状分析" §3): values is [rows][16] fp32; the row of
 *   raw id x is floor_mod(x, rows), i.e. the x % num_buckets of the page taken
 *   with Python semantics, always in [0, rows).  keys/digests/scores unused.
 *
 * kind == REC_HASH ("集成 DynamicEmb" §1, §3.2): a lookup-only open-addressing
 *   table of `rows` slots (the capacity), structure of arrays:
 *     keys[rows]     int64   stored key, or REC_EMPTY_KEY
 *     digests[rows]  uint8   0 exactly where the slot is empty, else digest(key)
 *     scores[rows]   uint64  carried for the owner, never read here (may be NULL)
 *     values[rows][16] fp32  the slot's embedding
 *   Placement convention (the builder must follow it): with
 *     h      = SplitMix64 output mix of the key's 64 bits (Steele, Lea, Flood,
 *              OOPSLA 2014; Stafford's Mix13 shifts 30/27/31 and multipliers
 *              0xbf58476d1ce4e5b9, 0x94d049bb133111eb),
 *     home   = floor(h * rows / 2^64),
 *     digest = h & 0xff, or 1 if that is 0,
 *   every stored key sits on the linear, wrapping probe sequence home,
 *   home+1, ... with no empty slot between its home and its slot.  A slot
 *   whose key was evicted (rec_hash_admit) holds REC_TOMBSTONE_KEY and keeps
 *   its nonzero digest: probes pass it.  A lookup of key x returns the slot
 *   holding x, or -1 (a miss) on reaching an empty slot or after `rows`
 *   probes; REC_EMPTY_KEY and REC_TOMBSTONE_KEY always miss.  A miss yields the zero vector
 *   (§3.2: the constant zero vector).  The raw id is the key (no modulo).
 *
 * Every table: dim == 16, rows >= 1 (REC_HASH: rows <= 2^31 - 1), values
 * 16-byte aligned (each row is 64 contiguous bytes); REC_HASH: digests
 * 16-byte aligned (the probe reads them 32 at a time), keys 8-byte aligned.
 */
typedef struct {
    int32_t kind;
    int32_t dim;
    int64_t rows;
    const float* values;
    const int64_t* keys;
    const uint8_t* digests;
    const uint64_t* scores;
} rec_table;

/*
 * Attention-MLP parameters for DIN ("当前现状分析" §4.2, §4.4; hidden units
 * [256, 64] as in "集成 DynamicEmb" §7), all device memory:
 *   w1 [256][192] (output-major, like torch.nn.Linear.weight), dtype `dtype`
 *      columns 0-47 q, 48-95 s, 96-143 q-s, 144-191 q*s; in each block the
 *      sub-features adgroup, cate, brand (16 each)
 *   b1 [256] fp32;  w2 [64][256] dtype `dtype`;  b2 [64] fp32
 *   w3 [64] fp32 (the 64 -> 1 score layer), b3 a host float
 * ReLU follows the 256- and 64-wide layers; the score has no activation.
 * dtype REC_BF16: w1/w2 are bf16 bit patterns.  The first layer is evaluated
 * through the identity W1 [q, s, q-s, q*s] = (W1q + W1d) q + (W1s - W1d) s +
 * W1m (q*s) (W1q, W1s, W1d, W1m its four 48-column blocks): the two column
 * sums are formed in fp32 and rounded to bf16 once; q, s and q*s (formed in
 * fp32) and the 256 hidden activations are rounded to bf16 (round to nearest
 * even) and multiplied on the matrix cores with fp32 accumulation; the
 * 64-wide layer, score, softmax and weighted sum stay fp32.
 * dtype REC_F32: every product and sum is fp32.
 * dtype REC_BF16_PACKED: as REC_BF16, but w1 points to the REC_DIN_PACKED_BYTES
 * image written by rec_din_pack_mlp (both layers, the first one factored, in
 * the order the attention kernel keeps them on chip) and w2 is not read.
 * Same results as REC_BF16.
 * w1 and w2 16-byte aligned.
 */
typedef struct {
    int32_t dtype;
    int32_t reserved;
    const void* w1;
    const float* b1;
    const void* w2;
    const float* b2;
    const float* w3;
    float b3;
} rec_din_mlp;

/*
 * Pre-pack the bf16 attention-MLP weights once (e.g. at model load) for the
 * attention kernel: reads mlp->w1 [256][192] and mlp->w2 [64][256] (dtype
 * REC_BF16, plain layout) and writes their matrix-core operand order into
 * `packed` (device, 16-byte aligned, >= REC_DIN_PACKED_BYTES bytes).  Use it
 * with dtype REC_BF16_PACKED.  W2 and W1m are copied unchanged; the blocks
 * W1q + W1d and W1s - W1d are formed in fp32 and rounded to bf16 (see
 * REC_BF16 above).
 * Errors: REC_EINVAL (null/misaligned pointers, dtype not REC_BF16),
 * REC_EWORKSPACE (packed_bytes too small).
 */
rec_status rec_din_pack_mlp(const rec_din_mlp* mlp, void* packed, size_t packed_bytes, void* stream);

/*
 * offsets = exclusive prefix sum of lengths ("当前现状分析" §2: a jagged
 * feature is values + lengths; offsets locate each bag/sequence).
 *   lengths  int32[n], each >= 0
 *   offsets  int64[n+1], 8-byte aligned: offsets[0] = 0, offsets[i+1] =
 *            offsets[i] + lengths[i]
 * No workspace: the per-block sums of the scan live in `offsets` itself until
 * the last of the call's three launches overwrites them.
 * Errors: REC_EINVAL (null lengths/offsets, n < 0, misaligned offsets).
 * n == 0 writes offsets[0] = 0 (one tiny kernel).
 */
rec_status rec_lengths_to_offsets(const int32_t* lengths, int64_t n, int64_t* offsets, void* stream);

/*
 * Sum-pooled embedding bags over T tables ("当前现状分析" §3, §4.4; DLRM
 * essay §3.2).  The KeyedJaggedTensor is key-major: bag i = t*B + b holds
 * values[offsets[i] .. offsets[i] + lengths[i]).
 *   tables   host array of T descriptors (table t pools feature t)
 *   values   int64[nnz] raw ids;  lengths int32[T*B];  offsets int64[T*B]
 *            (offsets[T*B] is not read)
 *   out      fp32 [B][T*16]: out[b][16t + d] = sum over bag (t, b) of row[d]
 *            (the KeyedTensor layout); an empty bag, and every hash miss,
 *            contributes +0.0; the sum runs in id order, fp32.  16-byte aligned.
 *   rows_out int64[nnz] or NULL: the resolved row of each id (REC_DIRECT: the
 *            floor-mod row; REC_HASH: the slot or -1)
 * Errors: REC_EINVAL (null pointers, T < 1, B < 0, bad table), REC_EUNSUPPORTED
 * (T > REC_MAX_TABLES).
 */
rec_status rec_embbag_fwd(const rec_table* tables, int32_t T, int64_t B,
                          const int64_t* values, const int32_t* lengths,
                          const int64_t* offsets, float* out, int64_t* rows_out,
                          void* stream);

/* Bytes of the KJT sums for T tables of B samples (about 0.26 B per bag); 0
 * for invalid arguments. */
size_t rec_kjt_sums_bytes(int32_t T, int64_t B);

/*
 * First half of the key-major offsets scan ("当前现状分析" §2), for callers
 * that hold only the KJT lengths: per table and 1024-sample block the block
 * sum, and per 32-sample chunk the chunk sum, written to `sums` (opaque,
 * >= rec_kjt_sums_bytes(T, B) bytes, 8-byte aligned).  rec_embbag_fwd_kjt
 * finishes the scan inside the embedding bags.
 *   lengths  int32[T*B], each >= 0
 * Errors: REC_EINVAL (null pointers, T < 1, B < 0, misalignment),
 * REC_EUNSUPPORTED (T > REC_MAX_TABLES), REC_EWORKSPACE.  B == 0 is a no-op.
 */
rec_status rec_kjt_sums(const int32_t* lengths, int32_t T, int64_t B, void* sums,
                        size_t sums_bytes, void* stream);

/*
 * rec_embbag_fwd for a KJT given by its lengths alone: each bag's offset is
 * derived on the device from `sums` (rec_kjt_sums of the same lengths, T and
 * B, earlier on the stream), so the offsets scan and the pooling take two
 * launches in all.  Same tables, values, lengths, out and rows_out as
 * rec_embbag_fwd, and bit-identical output.
 *   offsets_out int64[T*B+1] or NULL: the derived offsets (offsets[0] = 0,
 *               offsets[i+1] = offsets[i] + lengths[i])
 * Errors: as rec_embbag_fwd, plus REC_EINVAL (null or misaligned sums) and
 * REC_EWORKSPACE (sums_bytes too small).
 */
rec_status rec_embbag_fwd_kjt(const rec_table* tables, int32_t T, int64_t B,
                              const int64_t* values, const int32_t* lengths, const void* sums,
                              size_t sums_bytes, int64_t* offsets_out, float* out,
                              int64_t* rows_out, void* stream);

/*
 * Lookup-only hash probe ("集成 DynamicEmb" §3.2, §4.3) for n keys.
 *   table     host descriptor, kind REC_HASH
 *   keys      int64[n]
 *   slot_out  int64[n] or NULL: slot holding the key, or -1 on a miss
 *   rows_out  fp32 [n][16] or NULL: the slot's values, or 16 x +0.0 on a miss;
 *             16-byte aligned
 * At least one output must be non-NULL.
 * Errors: REC_EINVAL.
 */
rec_status rec_hash_lookup(const rec_table* table, const int64_t* keys, int64_t n,
                           int64_t* slot_out, float* rows_out, void* stream);

/* Bytes of workspace rec_hash_insert needs for n pairs into a table of
 * `capacity` slots (4 B per pair and 4 B per slot); 0 for n < 0, n > 2^30 or
 * a capacity outside [1, 2^31 - 1]. */
size_t rec_hash_insert_workspace_bytes(int64_t n, int64_t capacity);

/*
 * Insert-or-assign n (key, values) pairs into a hash table ("集成 DynamicEmb"
 * §6.4: a service rebuilds its tables at start-up by inserting the stored
 * key/value pairs; §4.2: score strategies; §1: the slot layout).  The
 * table's keys, digests, values (and scores) arrays are written.
 *   table      host descriptor, kind REC_HASH (the REC_HASH conditions above)
 *   keys       int64[n]
 *   values     fp32 [n][16], 16-byte aligned
 *   score_mode REC_SCORE_NONE: scores untouched (table->scores may be NULL);
 *              REC_SCORE_STEP: the slot's score becomes `step` (STEP evicts
 *              the oldest); REC_SCORE_LFU: the slot's score grows by one per
 *              insert (LFU evicts the least used); both need table->scores
 *   slot_out   int64[n] or NULL: the slot the key is stored in, -1 when the
 *              table had no empty slot on the key's probe sequence (the pair
 *              is not stored: no eviction, the NO_EVICTION behaviour), -2 for
 *              REC_EMPTY_KEY and REC_TOMBSTONE_KEY (never stored)
 *   workspace  >= rec_hash_insert_workspace_bytes(n, table->rows) bytes of
 *              device memory, 256-byte aligned, contents on entry ignored
 * The result is that of inserting the pairs one after another in index
 * order: a key already stored keeps its slot and gets the new values and
 * score; a new key takes an empty slot of its probe sequence, so the table
 * keeps the placement convention above; a key given several times in one
 * call is stored once, with the values of its last occurrence, and LFU counts
 * every occurrence.  Which empty slot a new key takes can depend on the order
 * in which concurrent lanes claim slots; every lookup result (found or not,
 * and the values) does not.  Nothing else may read or write the table while
 * the call runs.  Three launches.  Eviction and frequency admission are
 * rec_hash_admit's.
 * Errors: REC_EINVAL, REC_EUNSUPPORTED (n > 2^30), REC_EWORKSPACE.
 */
rec_status rec_hash_insert(const rec_table* table, const int64_t* keys, const float* values,
                           int64_t n, int32_t score_mode, uint64_t step, int64_t* slot_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace rec_hash_admit needs for n ids into a table of
 * `capacity` slots (about 40 B per id and 4 B per slot, plus 12.5 KiB for
 * the eviction's selection unless score_mode is REC_SCORE_NONE); 0 for
 * invalid arguments. */
size_t rec_hash_admit_workspace_bytes(int64_t n, int64_t capacity, int32_t score_mode);

/*
 * Frequency admission and score-driven eviction for one batch of ids
 * ("集成 DynamicEmb" §4.1: an id enters its table only once it has been seen
 * `threshold` times, and reads the constant 0 vector until then; §4.2: STEP
 * evicts the entry inserted earliest, LFU the one used least, NO_EVICTION
 * never evicts, so a full table stops taking ids; §2, §7: an initializer
 * gives a new row its values).  Rules, the ids of the call taken together:
 *   - every id counts once per occurrence; REC_EMPTY_KEY and
 *     REC_TOMBSTONE_KEY are ignored;
 *   - a stored id is used: REC_SCORE_STEP sets its score to `step`,
 *     REC_SCORE_LFU adds its occurrences; REC_SCORE_NONE (NO_EVICTION)
 *     leaves scores alone;
 *   - an id not stored adds its occurrences to its count in the counter
 *     table (0 when absent) and becomes a candidate when the count reaches
 *     `threshold`; otherwise the count is kept (a new id finding the counter
 *     table full is not counted);
 *   - the table holds at most max_keys ids.  Candidates are admitted in the
 *     order of their first occurrence while there is room.  For those left,
 *     STEP and LFU evict as many entries stored before the call, smallest
 *     score first (scores saturated at 2^32 - 2 for the comparison; equal
 *     scores: smaller id first, as signed integers), and admit as many more.
 *     Candidates not admitted keep their counts;
 *   - an evicted slot becomes a tombstone (key REC_TOMBSTONE_KEY, digest
 *     kept, score 0); lookups pass it, new ids may take it;
 *   - an admitted id takes an empty or tombstone slot of its probe sequence
 *     with no empty slot before it, its digest, its values from init_values
 *     at its first occurrence, the score `step` (STEP) or its count (LFU),
 *     and its count becomes 0.
 *   table        host descriptor, kind REC_HASH; keys, digests, values and (STEP,
 *                LFU) scores are written
 *   max_keys     0 .. capacity (capacity: the table may fill every slot)
 *   counter_keys int64[counter_capacity], counter_counts uint64[...]: the
 *                admission counters, kept by the caller across calls (start:
 *                keys REC_EMPTY_KEY, counts 0); placement by the table
 *                convention (no digests)
 *   keys         int64[n];  init_values fp32 [n][16], 16-byte aligned (e.g.
 *                N(0, 0.05) draws, the pages' initializer)
 *   slot_out     int64[n] or NULL: the slot of each id after the call, -1 if
 *                not stored, -2 for the reserved keys
 *   counts_out   device int64[3] or NULL: ids admitted, entries evicted,
 *                candidates left out
 *   workspace    >= rec_hash_admit_workspace_bytes(n, capacity, score_mode),
 *                256-byte aligned
 * Every stored value, count and score, the victims and the admitted ids are
 * the same run to run; which free slot a new id takes may depend on the order
 * of concurrent claims (no lookup result does), and so may which new ids get
 * a counter when the counter table overflows.  Nothing else may use the
 * tables during the call.  Seven launches, 20 with STEP or LFU (the 13
 * passes of the eviction's radix selection return at once when nothing is
 * evicted).  n == 0 is a no-op.
 * Errors: REC_EINVAL (null or misaligned arrays, bad table, score_mode,
 * max_keys, threshold 0), REC_EUNSUPPORTED (n > 2^30), REC_EWORKSPACE.
 */
rec_status rec_hash_admit(const rec_table* table, int64_t max_keys, int64_t* counter_keys,
                          uint64_t* counter_counts, int64_t counter_capacity, const int64_t* keys,
                          const float* init_values, int64_t n, uint64_t threshold, int32_t score_mode,
                          uint64_t step, int64_t* slot_out, int64_t* counts_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * DLRM dot-product interaction (DLRM essay, wmrh.cn/news/12459, §2.3: the
 * interaction layer takes the bottom MLP's output and every pooled embedding
 * and emits their pairwise dot products; §4.2: its code runs j from i, so the
 * diagonal is included; §3.1: measured at 217 features of width 96).
 *   z    fp32 [B][F][d], 16-byte aligned: sample b's F vectors (the bottom
 *        MLP's output first, then the pooled embeddings, in the caller's order)
 *   out  fp32 [B][F(F+1)/2]: out[b][p] = <z[b][i], z[b][j]> for the p-th pair
 *        i <= j in row order (0,0), (0,1), ..., (0,F-1), (1,1), ..., (F-1,F-1)
 * fp32 products with fp32 accumulation (on the matrix cores); the summation
 * order is not the sequential one, so results match an fp64 reference to a
 * few fp32 ulps of sum_k |z_ik z_jk|.
 * Limits: 1 <= F <= 256; d a multiple of 16, 16 <= d <= 512; the sample must
 * fit the kernel's LDS stage: 16 * ceil(F / 16) * (d + 4) * 4 bytes <= 144 KiB
 * (F = 217 allows d up to 160).
 * Errors: REC_EINVAL, REC_EUNSUPPORTED (shape beyond the limits).
 */
rec_status rec_dlrm_interact(const float* z, int64_t B, int32_t F, int32_t d, float* out, void* stream);

/*
 * The DLRM forward around the interaction (DLRM essay, wmrh.cn/news/12459:
 * §2.3 four layers -- a bottom MLP brings the dense features to the
 * embedding width, per-feature EmbeddingBags pool the sparse ids, the
 * interaction layer takes the dot product of every pair (one triangle only),
 * a top MLP turns the dot products into the prediction; §3.2 a bag pools by
 * sum or by mean; §3.3, §4.2 the widths and the pair order, j running from i;
 * §3.1 the measured interaction of 217 features of width 96).
 * For sample b:
 *   h     = relu(wb2 relu(wb1 dense[b] + bb1) + bb2)        (d)
 *   e_t   = sum over bag (t, b) of table t's rows (REC_POOL_SUM), or that sum
 *           divided by the bag's length (REC_POOL_MEAN); an empty bag gives 0
 *   z[b]  = [h, e_0, ..., e_{S-1}]                         ([S+1][d])
 *   I     = <z_i, z_j> for i <= j in row order (0,0), (0,1), ..., (S,S)
 *   logit = wt3 . relu(wt2 relu(wt1 I + bt1) + bt2) + bt3;  prob = sigmoid
 * All fp32; each dot product and layer sums in a fixed order (results are
 * bit-identical run to run).
 */
typedef struct {
    int32_t n_dense;              /* dense features, 1..128 */
    int32_t dim;                  /* d: table width = bottom output, 32..256, multiple of 32 */
    int32_t S;                    /* sparse features (tables), 1..255 */
    int32_t reserved;
    const float* wb1;             /* [128][n_dense] (torch.nn.Linear.weight layout) */
    const float* bb1;             /* [128] */
    const float* wb2;             /* [dim][128] */
    const float* bb2;             /* [dim] */
    const float* wt1;             /* [128][(S+1)(S+2)/2] */
    const float* bt1;             /* [128] */
    const float* wt2;             /* [64][128] */
    const float* bt2;             /* [64] */
    const float* wt3;             /* [64] */
    float bt3;
} rec_dlrm_mlp;

/*
 *   mlp      host struct; every array 16-byte aligned device memory
 *   tables   host array of S descriptors, kind REC_DIRECT, dim == mlp->dim
 *            (values [rows][dim] fp32, 16-byte aligned); row = floor_mod(id, rows)
 *   modes    host int32[S]: REC_POOL_SUM or REC_POOL_MEAN per table
 *   dense    fp32 [B][n_dense]
 *   values   int64[nnz] ids;  lengths int32[S*B];  offsets int64[S*B]: the
 *            key-major KJT (bag t*B + b holds values[offsets[t*B+b] .. +
 *            lengths[t*B+b])), e.g. from rec_lengths_to_offsets
 *   z        fp32 [B][S+1][dim], 16-byte aligned: written (the interaction
 *            input: bottom output first, then the bags in table order)
 *   inter    fp32 [B][(S+1)(S+2)/2] or NULL: the interaction output (required
 *            for a wide model, below)
 *   logit    fp32 [B];  prob fp32 [B] or NULL
 * S <= 31 and (S+1)*dim <= 1024: one launch, z held on chip per workgroup.
 * Otherwise (a wide model, e.g. 216 tables of width 96: the 217-feature
 * interaction) z and the interaction output go through memory: the bags
 * (one launch per 32 tables), the bottom MLP, the interaction (as
 * rec_dlrm_interact, whose limits apply: 32 * ceil((S+1)/32) rows of about
 * dim + 4 floats within 144 KiB, e.g. dim <= 160 at S = 216) and the top MLP.
 * Errors: REC_EINVAL (null required pointers, misalignment, B < 0, a table
 * that is not direct or whose dim differs, unknown mode, sizes outside the
 * limits above, inter NULL for a wide model), REC_EUNSUPPORTED (a wide model
 * beyond the interaction's LDS stage).  B == 0 is a no-op.
 */
rec_status rec_dlrm_fwd(const rec_dlrm_mlp* mlp, const rec_table* tables, const int32_t* modes,
                        int64_t B, const float* dense, const int64_t* values,
                        const int32_t* lengths, const int64_t* offsets, float* z, float* inter,
                        float* logit, float* prob, void* stream);

/*
 * Empties a hash table: every key becomes REC_EMPTY_KEY, every digest 0 and
 * every score 0 (when table->scores is not NULL); values are left as they
 * are.  The start of a rebuild ("集成 DynamicEmb" §6.4).
 * Errors: REC_EINVAL.
 */
rec_status rec_hash_clear(const rec_table* table, void* stream);

/* Bytes of the DIN plan buffer for B samples capped at max_len positions
 * (about 20 bytes per possible position, B * max_len, plus per-sample data);
 * 0 for invalid arguments. */
size_t rec_din_plan_bytes(int64_t B, int32_t max_len);

/*
 * Sequence side of the forward, before the attention ("当前现状分析" §4.1:
 * real lengths are ~3-5 of a cap of 100, so positions are packed, not padded;
 * §3 / "集成 DynamicEmb" §3.2 for the id -> row rule).  On the device it
 *   - packs the positions: sample b, step j < L_b = min(seq_lengths[b],
 *     max_len) becomes packed position pos_start(b) + j, where pos_start is
 *     the exclusive prefix sum of the L_b;
 *   - records how rec_din_attn_fwd_plan splits the P = sum L_b packed positions
 *     over its waves: ranges of `range_positions` positions (0 = P split
 *     evenly over every wave the device runs at once, rounded up to 16);
 *   - resolves the three sub-feature ids of every packed position to its row
 *     (direct: floor modulo; hash: probe, -1 on a miss).
 * Inputs:
 *   seq_tables  host array of 3 descriptors (adgroup, cate, brand); each at
 *               most 2^31 - 1 rows
 *   seq_values  int64 [3][seq_stride]: sub-feature f's id at step j of sample b
 *               is seq_values[f*seq_stride + off_b + j]
 *   seq_offsets int64[B] giving off_b (any layout, e.g. padded off_b = 100 b),
 *               or NULL for the packed jagged layout (off_b = exclusive prefix
 *               sum of the unclamped seq_lengths)
 *   seq_lengths int32[B], each >= 0
 * Outputs:
 *   plan            >= rec_din_plan_bytes(B, max_len) bytes, 16-byte aligned,
 *                   opaque; used by rec_din_attn_fwd_plan
 *   seq_offsets_out int64[B+1] or NULL: exclusive prefix sum of the unclamped
 *                   seq_lengths (the jagged offsets)
 *   rows_out        int64 [3][seq_stride] or NULL: the row/slot of every id
 *                   read (positions past L_b are never read or written)
 * Errors: REC_EINVAL (null seq_tables/seq_values/seq_lengths/plan, bad table,
 * B < 0, max_len outside [1, REC_MAX_SEQ_LEN], range_positions not 0 or a
 * multiple of 16 in [16, 2^20]), REC_EUNSUPPORTED (B > REC_MAX_B, a table
 * above 2^31 - 1 rows), REC_EWORKSPACE.
 */
rec_status rec_din_plan(const rec_table* seq_tables, const int64_t* seq_values,
                        int64_t seq_stride, const int64_t* seq_offsets,
                        const int32_t* seq_lengths, int64_t B, int32_t max_len,
                        int32_t range_positions, int64_t* seq_offsets_out, int64_t* rows_out,
                        void* plan, size_t plan_bytes, void* stream);

/* Bytes of workspace rec_din_attn_fwd needs for B samples capped at max_len
 * positions (the plan it builds: about 20 bytes per possible position,
 * B * max_len, plus per-sample data); 0 for invalid arguments. */
size_t rec_din_attn_workspace_bytes(int64_t B, int32_t max_len);

/*
 * DIN target attention, padding-free, in one call ("当前现状分析" §4.2: the
 * attention input [q, s, q-s, q*s], attn MLP (256, 64), one score per
 * position, masked softmax, weighted sum; §4.4: query [B,48], output [B,48];
 * §4.1: real lengths are ~3-5 of a cap of 100, so positions are packed, never
 * padded; §6.4 of the same page: the sparse model hands over the query, the
 * sequence and its lengths).  For sample b with L_b = min(seq_lengths[b],
 * max_len) positions j < L_b:
 *   s_j = [adgroup row | cate row | brand row] of the ids
 *         seq_values[f*seq_stride + off_b + j], f = 0..2, in seq_tables[f]
 *         (direct: floor-mod row; hash: the slot, a miss reads 16 x +0.0)
 *   q   = query[b*query_ld + query_col[f] + d] (f = 0..2, d < 16), the pooled
 *         target features (for rec_embbag_fwd's output with the 16 deep
 *         features in page order: query_ld 256, query_col {16, 80, 48})
 *   e_j = w3 . relu(W2 relu(W1 [q, s_j, q - s_j, q*s_j] + b1) + b2) + b3
 *   p_j = softmax over j < L_b of e_j (max-subtracted, no temperature)
 *   out[b][0..48) = sum_j p_j s_j;  L_b == 0 gives 48 x +0.0
 * Positions j >= L_b are never read, so any sequence layout with the same
 * lengths gives bit-identical output.  P = sum_b L_b is the number of packed
 * positions; packed position pos_start(b) + j (pos_start = exclusive prefix
 * sum of the L_b) indexes scores_out and weights_out.
 *   seq_tables  host array of 3 descriptors (adgroup, cate, brand), each at
 *               most 2^31 - 1 rows
 *   seq_values  int64 [3][seq_stride] raw ids
 *   seq_offsets int64[B] giving off_b (any layout, e.g. padded off_b = 100 b),
 *               or NULL for the packed jagged layout (off_b = exclusive prefix
 *               sum of the unclamped seq_lengths)
 *   seq_lengths int32[B], each >= 0;  max_len in [1, REC_MAX_SEQ_LEN]
 *   query       fp32, rows 16-byte aligned (query_ld and query_col[f]
 *               multiples of 4);  query_col host int32[3]
 *   mlp         host struct (device arrays inside)
 *   out         fp32 [B][48], 16-byte aligned
 *   scores_out  fp32 [P] or NULL: e at each packed position
 *   weights_out fp32 [P] or NULL: p at each packed position (needs scores_out)
 *   rows_out    int64 [3][seq_stride] or NULL: the row/slot (-1: hash miss) of
 *               every id read (positions past L_b are not written)
 *   workspace   >= rec_din_attn_workspace_bytes(B, max_len) bytes of device
 *               memory, 16-byte aligned, contents on entry ignored; it holds
 *               the plan (packed positions, resolved rows, work split)
 * Three launches: plan sums, plan build, attention.  A sample whose positions
 * the attention splits between two waves is merged from their partial sums,
 * so a device with another number of compute units may change the last bits
 * of its output (not of scores_out).
 * Errors: REC_EINVAL (null seq_tables/seq_values/seq_lengths/query/query_col/
 * mlp/out, bad table or mlp, misalignment, B < 0, max_len outside
 * [1, REC_MAX_SEQ_LEN], weights_out without scores_out), REC_EUNSUPPORTED
 * (B > REC_MAX_B, a sequence table above 2^31 - 1 rows), REC_EWORKSPACE
 * (workspace NULL or smaller than required).  B == 0 is a no-op.
 */
rec_status rec_din_attn_fwd(const rec_table* seq_tables, const int64_t* seq_values,
                            int64_t seq_stride, const int64_t* seq_offsets,
                            const int32_t* seq_lengths, int32_t max_len, int64_t B,
                            const float* query, int64_t query_ld, const int32_t* query_col,
                            const rec_din_mlp* mlp, float* out, float* scores_out,
                            float* weights_out, int64_t* rows_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * The attention of rec_din_attn_fwd over a plan built earlier by
 * rec_din_plan (same seq_tables, B and max_len), for callers that build the
 * plan on another stream or reuse it: out, scores_out and weights_out are
 * those of rec_din_attn_fwd; a plan with range_positions != 0 splits the
 * positions differently, which may change the last bits of a sample cut
 * between waves.  The plan is only read.  One launch.
 * Errors: as rec_din_attn_fwd, with REC_EWORKSPACE for a missing plan or one
 * smaller than rec_din_plan_bytes(B, max_len).
 */
rec_status rec_din_attn_fwd_plan(const rec_table* seq_tables, const void* plan, size_t plan_bytes,
                                 int64_t B, int32_t max_len, const float* query, int64_t query_ld,
                                 const int32_t* query_col, const rec_din_mlp* mlp, float* out,
                                 float* scores_out, float* weights_out, void* stream);

/*
 * The whole sparse forward in one call: rec_kjt_sums + rec_din_plan +
 * rec_embbag_fwd_kjt + rec_din_attn_fwd_plan, with the query read from the pooled
 * output.  The deep and sequence sides share launches (three in all instead
 * of five).  Results are bit-identical to the four calls made one by one.
 * Every pointer is a device pointer except `tables`, `seq_tables` and `mlp`
 * (host); arrays are as the four calls document them.
 */
typedef struct {
    int32_t T;                    /* deep tables, 1..REC_MAX_TABLES */
    int32_t max_len;              /* sequence cap, 1..REC_MAX_SEQ_LEN */
    int64_t B;                    /* samples, 0..REC_MAX_B */
    const rec_table* tables;      /* host [T] */
    const int64_t* values;        /* [nnz] key-major raw ids */
    const int32_t* lengths;       /* [T*B] */
    const rec_table* seq_tables;  /* host [3]: adgroup, cate, brand */
    const int64_t* seq_values;    /* [3][seq_stride] */
    int64_t seq_stride;
    const int64_t* seq_offsets;   /* [B], or NULL for the packed jagged layout */
    const int32_t* seq_lengths;   /* [B] */
    int32_t query_col[3];         /* pooled columns of the query (16 k per table k) */
    int32_t range_positions;      /* as rec_din_plan; 0 = even split */
    const rec_din_mlp* mlp;       /* host */
    float* pooled;                /* [B][T*16], 16-byte aligned */
    float* att;                   /* [B][48], 16-byte aligned */
    int64_t* offsets_out;         /* [T*B+1] or NULL */
    int64_t* rows_out;            /* [nnz] or NULL */
    int64_t* seq_offsets_out;     /* [B+1] or NULL */
    int64_t* seq_rows_out;        /* [3][seq_stride] or NULL */
    float* scores_out;            /* [P] or NULL */
    float* weights_out;           /* [P] or NULL (needs scores_out) */
    void* workspace;              /* >= rec_sparse_din_fwd_workspace_bytes, 16-byte aligned */
    size_t workspace_bytes;
} rec_fwd_args;

/* Workspace bytes of rec_sparse_din_fwd (KJT sums + plan); 0 for invalid
 * arguments. */
size_t rec_sparse_din_fwd_workspace_bytes(int32_t T, int64_t B, int32_t max_len);

/* Errors: those of the four calls (messages name rec_sparse_din_fwd), plus
 * REC_EINVAL (args or workspace NULL or misaligned) and REC_EWORKSPACE.
 * B == 0 is a no-op. */
rec_status rec_sparse_din_fwd(const rec_fwd_args* args, void* stream);

/*
 * rec_sparse_din_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same forward, kernels and results, with the workspace
 * (KJT sums and plan) in a static device array of REC_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds on each device it runs on, from load until
 * the process ends.  args->workspace and args->workspace_bytes are ignored;
 * the caller still passes every input and output.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up the array's address there.
 * Every call on one device shares that device's array and leaves its
 * contents behind: calls that overlap on one device (on two streams, or from
 * two threads without ordering) race and give undefined results.  Nothing in
 * the array needs to start at zero.
 * Limit: rec_sparse_din_fwd_workspace_bytes(T, B, max_len) must not exceed
 * REC_NOALLOC_SCRATCH_BYTES (at T = 16, max_len = 100: B up to about 16,000;
 * the Taobao batch, B = 8192, needs about 16.6 MB).
 * Errors: those of rec_sparse_din_fwd (messages name
 * rec_sparse_din_fwd_noalloc), with REC_EWORKSPACE for a batch beyond the
 * limit (checked before anything else; no device is touched).
 */
rec_status rec_sparse_din_fwd_noalloc(const rec_fwd_args* args, void* stream);

/*
 * The rest of the MultiTowerDIN forward after the sparse part: the deep tower
 * and the final MLP ("当前现状分析" §4.4 compute graph: deep MLP
 * 512 -> 256 -> 128 over the pooled deep features, concat with the [B,48]
 * attention output into [B,176], final MLP 176 -> 64 -> 1; "集成 DynamicEmb"
 * §7 model config: tower hidden units [512, 256, 128], final [64], binary
 * cross entropy, so the last unit is a logit):
 *   d1 = relu(wd1 x + bd1)   x = pooled[b][0..255]       wd1 [512][256]
 *   d2 = relu(wd2 d1 + bd2)                              wd2 [256][512]
 *   d3 = relu(wd3 d2 + bd3)  -> deep_out[b]              wd3 [128][256]
 *   f  = relu(wf [d3, att[b]] + bf)                      wf  [64][176]
 *   logit[b] = wo . f + bo;  prob[b] = 1 / (1 + exp(-logit[b]))
 * Matrices are output-major (torch.nn.Linear.weight), dtype `dtype`; biases
 * and wo are fp32; bo is a host float.  In the concat the deep output comes
 * first (wf columns 0-127), then att (columns 128-175).
 * dtype REC_BF16: the inputs (pooled, att) and every hidden activation are
 * rounded to bf16 (nearest even) and multiplied on the matrix cores with
 * fp32 accumulation; biases, the 64 -> 1 logit and the logistic are fp32;
 * deep_out is d3 before its bf16 rounding.  dtype REC_F32: fp32 throughout.
 * dtype REC_BF16_PACKED: as REC_BF16, but wd1 points to the
 * REC_TOWER_PACKED_BYTES image written by rec_tower_pack_mlp (all four
 * matrices in the order the kernel reads them) and wd2, wd3, wf are not read.
 * Same results as REC_BF16, several times faster.
 */
typedef struct {
    int32_t dtype;                /* REC_F32, REC_BF16 or REC_BF16_PACKED */
    int32_t reserved;
    const void* wd1;
    const float* bd1;
    const void* wd2;
    const float* bd2;
    const void* wd3;
    const float* bd3;
    const void* wf;
    const float* bf;
    const float* wo;
    float bo;
} rec_tower_mlp;

/*
 *   mlp       host; every array 16-byte aligned device memory
 *   pooled    fp32 [B][pooled_ld], pooled_ld >= 256 and a multiple of 4; the
 *             first 256 columns are the deep input (16 tables x 16)
 *   att       fp32 [B][48] (rec_din_attn_fwd's output)
 *   deep_out  fp32 [B][128] or NULL;  logit fp32 [B];  prob fp32 [B] or NULL
 * pooled, att and deep_out 16-byte aligned.
 * Errors: REC_EINVAL (null required pointers, bad dtype, misalignment,
 * pooled_ld, B < 0).  B == 0 is a no-op.
 */
rec_status rec_towers_fwd(const rec_tower_mlp* mlp, int64_t B, const float* pooled,
                          int64_t pooled_ld, const float* att, float* deep_out, float* logit,
                          float* prob, void* stream);

/*
 * Pre-pack the bf16 tower matrices once (e.g. at model load): reads wd1,
 * wd2, wd3 and wf of `mlp` (dtype REC_BF16, plain layout) and writes their
 * matrix-core operand order into `packed` (device, 16-byte aligned,
 * >= REC_TOWER_PACKED_BYTES bytes; wf's columns are padded to 192 with
 * zeros).  Use it with dtype REC_BF16_PACKED.  The values are copied
 * unchanged.  Errors: REC_EINVAL (null/misaligned pointers, dtype not
 * REC_BF16), REC_EWORKSPACE (packed_bytes too small).
 */
rec_status rec_tower_pack_mlp(const rec_tower_mlp* mlp, void* packed, size_t packed_bytes,
                              void* stream);

/*
 * One table as the sparse AdaGrad step sees it (host struct; the arrays are
 * device memory; weights and accum are updated in place).
 *   weights  fp32 [rows][16], 16-byte aligned: the table rec_embbag_fwd reads
 *            (REC_HASH: the slot values)
 *   accum    fp32 [rows][16], 16-byte aligned: AdaGrad's running sum of
 *            squared gradients, one value per weight (0 before the first step)
 *   rows     REC_DIRECT: num_buckets, the floor-mod divisor; REC_HASH: the
 *            capacity
 *   kind     REC_DIRECT or REC_HASH;  keys, digests: REC_HASH only, laid out
 *            and aligned as in rec_table (a read of a key no slot holds is a
 *            miss, which read the zero vector and takes no gradient)
 */
typedef struct {
    float* weights;
    float* accum;
    int64_t rows;
    int32_t kind;
    int32_t reserved;
    const int64_t* keys;
    const uint8_t* digests;
} rec_adagrad_table;

/* Bytes of workspace rec_embbag_adagrad needs for T tables, B samples, nnz
 * bag ids and P sequence positions (about 25 B per read: 16 B of keys and
 * sources, 8 B of partial sums, 1 B of digit counts); 0 for invalid
 * arguments or nnz + P == 0. */
size_t rec_embbag_adagrad_workspace_bytes(int32_t T, int64_t B, int64_t nnz, int64_t P);

/*
 * Backward of the sum-pooled embedding bags (and of the unpooled sequence
 * rows the DIN attention reads) followed by one sparse AdaGrad step
 * ("当前现状分析": the run-config table trains sparse parameters with
 * AdaGrad, lr 1e-3, and §3 sizes its accumulator like the table; "集成
 * DynamicEmb" §3.3: gradients accumulate in fp32).
 *
 * Gradient of each row: the sum, over every read of that row in the batch, of
 * the read's output gradient:
 *   - id i of bag (t, b) (the KJT of rec_embbag_fwd: key-major, bag t*B + b
 *     holds values[offsets[t*B+b] .. + lengths[t*B+b])) reads the row of
 *     values[i] in table t (REC_DIRECT: floor_mod(values[i], rows); REC_HASH:
 *     the slot holding it, none on a miss), with output gradient
 *     grad_pooled[b][16t .. 16t+16);
 *   - packed sequence position j < P of sub-feature k (0..2) reads the row of
 *     seq_values[k*seq_stride + j] in table seq_table[k], with output gradient
 *     grad_seq[k][j][0..16).
 * Every row read at least once then takes, element by element, with its
 * summed gradient g:  accum += g*g;  weights -= lr * g / (sqrt(accum) + eps)
 * (fp32).  Rows not read are not touched.  A repeated id counts once per
 * repetition.  The sums run in a fixed order (reads sorted by row with a
 * stable radix sort, no atomics), so results are bit-identical run to run.
 *
 *   tables      host array of T rec_adagrad_table (T <= REC_MAX_TABLES),
 *               direct or hash; rows summing to less than 2^32 - 1
 *   values      int64[nnz] raw ids; lengths int32[T*B]; offsets int64[T*B]:
 *               the exclusive scan of lengths, with offsets[T*B-1] +
 *               lengths[T*B-1] == nnz (precondition, not checked)
 *   grad_pooled fp32 [B][T*16], 16-byte aligned
 *   seq_table   host int32[3] (table index of each sub-feature), or NULL when
 *               P == 0;  seq_values int64 [3][seq_stride], seq_stride >= P;
 *   grad_seq    fp32 [3][P][16], 16-byte aligned (NULL when P == 0)
 *   lr, eps     the step size and the denominator's epsilon (e.g. 1e-3, 1e-10)
 *   workspace   >= rec_embbag_adagrad_workspace_bytes(T, B, nnz, P) bytes of
 *               device memory, 256-byte aligned; contents on entry ignored
 * The tables must not overlap one another or the inputs.
 * Errors: REC_EINVAL (null or misaligned pointers, T < 1, B < 0, nnz < 0,
 * P < 0, rows < 1, unknown kind, a hash table without keys or digests, a
 * seq_table entry outside [0, T)), REC_EUNSUPPORTED (T > REC_MAX_TABLES, rows
 * summing to 2^32 - 1 or more, nnz + 3P or B*T + 3P at 2^31 or more),
 * REC_EWORKSPACE.  nnz + P == 0 is a no-op.
 */
rec_status rec_embbag_adagrad(const rec_adagrad_table* tables, int32_t T, int64_t B,
                              const int64_t* values, const int32_t* lengths,
                              const int64_t* offsets, int64_t nnz, const float* grad_pooled,
                              const int32_t* seq_table, const int64_t* seq_values,
                              int64_t seq_stride, int64_t P, const float* grad_seq, float lr,
                              float eps, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace rec_din_attn_bwd needs: 256 KiB (the transposed
 * weights) plus about 3.7 KiB per position index (seq_stride), and 64 MiB more
 * with weight gradients. */
size_t rec_din_attn_bwd_workspace_bytes(int64_t seq_stride, int32_t weight_grads);

/*
 * Backward of the DIN target attention ("当前现状分析" §4.2, §4.4: the
 * forward [q, s, q-s, q*s] -> attn MLP (256, 64) -> score -> masked softmax
 * -> weighted sum of the sequence rows; the run-config table's training step
 * through it).  Given grad_att = dL/d att [B][48], computes by the chain rule
 * (the forward is recomputed from the same inputs rec_din_attn_fwd takes):
 *   grad_query [B][48]        dL/dq (for the pooled columns query_col[k] .. +16
 *                             of the sample's deep bags; the caller adds it to
 *                             the pooled gradient)
 *   grad_seq [3][seq_stride][16] or NULL: dL/ds for every position index
 *                             seq_offsets[b] + j, j < min(len_b, max_len);
 *                             every other index gets zeros (rec_embbag_adagrad
 *                             takes it as its sequence gradient)
 *   dw1 [256][192], db1 [256], dw2 [64][256], db2 [64], dw3 [64], db3 [1]
 *                             all six, or all NULL (no weight gradients): the
 *                             sums over every sample and position
 * Inputs as rec_din_attn_fwd: seq_tables host [3] (adgroup, cate, brand;
 * direct or hash, a miss reads the zero vector), seq_values int64
 * [3][seq_stride], seq_offsets int64 [B] (first position index of sample b;
 * required, and the samples' position ranges [off_b, off_b + L_b) must not
 * overlap: per-position data lives at the position index, so two samples
 * sharing one would overwrite each other's terms -- precondition, not
 * checked),
 * seq_lengths int32 [B], max_len in [1, REC_MAX_SEQ_LEN], query fp32 with row
 * stride query_ld and host query_col[3]; mlp host, dtype REC_F32 or REC_BF16
 * (plain layout; b1 and b2 may be NULL for zero biases).  The arithmetic is
 * fp32; sums run in one fixed order (bit-identical run to run).
 *   workspace  >= rec_din_attn_bwd_workspace_bytes(seq_stride, weight grads
 *              requested) bytes, 256-byte aligned
 * Errors: REC_EINVAL (null required pointers, misalignment, B < 0, bad
 * max_len or query_col, some but not all weight-gradient pointers, bad
 * table), REC_EUNSUPPORTED (dtype REC_BF16_PACKED), REC_EWORKSPACE.  B == 0 is
 * a no-op.
 */
rec_status rec_din_attn_bwd(const rec_table* seq_tables, const int64_t* seq_values,
                            int64_t seq_stride, const int64_t* seq_offsets,
                            const int32_t* seq_lengths, int32_t max_len, int64_t B,
                            const float* query, int64_t query_ld, const int32_t* query_col,
                            const rec_din_mlp* mlp, const float* grad_att, float* grad_query,
                            float* grad_seq, float* dw1, float* db1, float* dw2, float* db2,
                            float* dw3, float* db3, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Measurement hook: the next launch, made by this thread through any entry
 * point, of the kernel named by `kernel` records hipEvent_t `start` when that
 * kernel begins and `stop` when it ends (the events are bound to the kernel's
 * dispatch, hipExtLaunchKernelGGL), so hipEventElapsedTime(start, stop) is the
 * kernel's own execution time, as a kernel trace measures it, without the
 * launch's dispatch gap.  Kernels:
 *   REC_TIME_DIN_ATTN       the DIN attention (rec_din_attn_fwd,
 *                           rec_din_attn_fwd_plan, rec_sparse_din_fwd)
 *   REC_TIME_GATHER         the embedding bags (rec_embbag_fwd,
 *                           rec_embbag_fwd_kjt) or, in rec_sparse_din_fwd, the
 *                           launch that builds the plan and pools the bags
 *   REC_TIME_SUMS           the KJT sums (rec_kjt_sums; with the plan sums in
 *                           rec_sparse_din_fwd)
 *   REC_TIME_TOWERS         the bf16 towers (rec_towers_fwd)
 *   REC_TIME_DLRM_INTERACT  the interaction (rec_dlrm_interact)
 *   REC_TIME_DLRM_FWD       rec_dlrm_fwd's launch (for a wide model, the last
 *                           of its launches: the top MLP)
 * The events (created by the caller with timing enabled, on the device of
 * the launch) are used by one launch and then forgotten; start == stop ==
 * NULL forgets them without a launch.  The setting is thread-local state of
 * the library.  Not for use while a stream is being captured into a graph.
 * Errors: REC_EINVAL (unknown kernel, one event NULL and not the other).
 */
rec_status rec_time_next_launch(int32_t kernel, void* start, void* stop);

/* Message for the last non-OK status on this thread ("" if none). */
const char* rec_last_error(void);

/* ABI version (major*100 + minor). */
int32_t rec_version(void);

/*
 * Host-side twins of the device index arithmetic, for testing that
 * arithmetic without a GPU: the same inline functions the kernels run.
 *   rec_host_floor_mod: row of raw id x in a direct table of n rows (n >= 1)
 *   rec_host_hash_home: home slot of key x in a table of `capacity` slots;
 *                       *digest receives the key's digest byte
 *   rec_host_hash_probe: the slot holding `key` in a hash table given by its
 *                       host arrays keys[capacity] and digests[capacity]
 *                       (16-byte aligned), -1 if absent, -2 for invalid
 *                       arguments: the device's windowed probe, run on the host
 */
int64_t rec_host_floor_mod(int64_t x, int64_t n);
int64_t rec_host_hash_home(int64_t x, int64_t capacity, uint8_t* digest);
int64_t rec_host_hash_probe(const int64_t* keys, const uint8_t* digests, int64_t capacity,
                            int64_t key);

#ifdef __cplusplus
}
#endif

#endif /* REC_H */
