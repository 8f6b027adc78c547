/*
 * gqa_decode.h -- single-token GQA flash-decode attention over a bf16 KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * Computes, for every sequence b and query head h,
 *
 *     out[b,h,:] = softmax(scale * q[b,h,:] . K[b,h/G,0:len,:]^T) . V[b,h/G,0:len,:]
 *
 * with G = Hq / Hkv query heads per kv head (grouped consecutively: query
 * head h reads kv head h / G) and len = seq_lens[b].  The KV range of every
 * (sequence, kv head) is cut into splits; each split emits unnormalised
 * partials (m, l, acc) that a combine step folds with the log-sum-exp rescale
 * in a fixed order (sparkinfer PR #877 "split the flash-decode KV range
 * across warp-groups", section Mechanism; AstrAI csrc commit log, the split-KV
 * decode bullets: partials over gridDim.z blocks reduced by a combine kernel,
 * split count chosen to fill the device).  All G query heads of a kv head are
 * computed by one workgroup, so each K/V byte is read from HBM once (AstrAI
 * csrc commit log, the decode MMA head-packing bullets).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are caller-owned DEVICE memory.  q, k, v, out and
 *     workspace must be 16-byte aligned; seq_lens and page_table 4-byte
 *     aligned.  bf16 tensors are passed as raw 16-bit patterns (E4M3 caches
 *     as raw bytes, see gqa_decode_fp8).
 *   - Calls only enqueue work on `stream` (0 = the null stream): they never
 *     synchronise and never allocate device memory.  The library keeps no
 *     state besides a cached CU count and the kernels' function handles per
 *     device, the process-wide tuning (gqa_tuning_t) and the static scratch
 *     array of gqa_decode_noalloc.  Outputs are ready when
 *     the stream reaches them.
 *   - Every argument check runs on the host before any launch; a rejected call
 *     launches nothing and returns the status below.  A failed launch returns
 *     GQA_ERR_HIP.  Nothing throws across this interface.
 *   - Device-resident preconditions that the host cannot check:
 *     0 <= seq_lens[b] <= capacity, and (paged) page_table[b][i] in
 *     [0, num_pages) for i < ceil(seq_lens[b] / page_size).  Entries past that
 *     are never read.  A sequence of length 0 yields a zero output row.
 *     Out-of-range lengths and page ids are clamped on the device so that no
 *     access leaves the buffers; the output for such inputs is unspecified.
 *   - B = 0 is a no-op that reads no pointer (they may be NULL).
 *   - Results are bit-identical from run to run for the same inputs, device
 *     and plan (fixed fold orders, no atomics in the arithmetic).  Different
 *     split counts re-associate the sums and may differ in the last bits.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_NULL = 1,        /* a required pointer is NULL */
    GQA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    GQA_ERR_UNSUPPORTED = 3, /* head_dim not in {32,64,128,256} (E4M3: {64,128,256}), G > 16, page_size % 16 != 0 */
    GQA_ERR_ALIGN = 4,       /* a pointer violates the alignment above */
    GQA_ERR_WORKSPACE = 5,   /* workspace smaller than the plan needs */
    GQA_ERR_HIP = 6,         /* a HIP runtime call or launch failed */
    GQA_ERR_TOO_LARGE = 7    /* gqa_decode_noalloc: the call needs more scratch than its static buffer */
} gqa_status_t;

/* How a call is laid out on the device (host-side, deterministic). */
typedef struct gqa_plan {
    int partition;          /* 0: fixed splits per (sequence, kv head); 1: even shares;
                               2: proportional splits (gqa_tuning_t.partition = 3) */
    int num_splits;         /* fixed: S, KV partitions per (sequence, kv head); even: 0 */
    int split_tokens;       /* fixed: keys per split; even: keys per share at full length */
    int tile_tokens;        /* keys one wave stages per pipeline step */
    int waves;              /* waves (of 64 lanes) per workgroup */
    int grid;               /* workgroups of the split kernel: B * Hkv * S, or the shares */
    int direct;             /* 1: S == 1, the split kernel writes `out` itself */
    int max_pieces;         /* most partials one (sequence, kv head) has with every sequence at full
                               length (even shares: shorter sequences elsewhere can give more) */
    int64_t slots;          /* partial blocks in the workspace: B*Hkv*S, or shares + B*Hkv */
    int pv_mode;            /* PV contraction: 1 = bf16 MFMA with P split hi+lo, 0 = fp32 MFMA */
    int double_buffer;      /* 1: two tile buffers per wave; 0: one, refilled part by part */
    int streaming;          /* 1: K/V loads carry the non-temporal hint (large caches) */
    size_t workspace_bytes; /* scratch the call needs (0 when direct) */
    int fused;              /* 1: the split kernel folds its own partials (one launch, see gqa_tuning_t.fold);
                               0: a combine kernel folds them (two launches) */
    int fold_fanin;         /* fused fixed splits: partials per node of the fold tree; otherwise 0 */
    int64_t counters;       /* arrival counters a fused call uses in the workspace header (0 otherwise) */
    int qk_mode;            /* QK^T contraction: 0 = bf16 MFMA, 1 = vector ALU (see gqa_tuning_t.qk_mode) */
} gqa_plan_t;

/*
 * Tuning: the plan and kernel-variant choices every call makes, process-wide.
 * The defaults (gqa_decode_get_tuning right after loading, when no GQA_DECODE_*
 * variable is set) are the measured best on MI355X.  The environment
 * variables named below override single fields for same-binary A/B runs; they
 * are read ONCE, when the library is loaded, never per call.
 * gqa_decode_set_tuning replaces the whole set at run time (thread-safe).
 * Every call copies the tuning once at entry, so the launches of one call and
 * the plan they follow always agree.  A *_partials call and the
 * gqa_decode_combine that folds its partials must run under the same tuning.
 */
typedef struct gqa_tuning {
    int tile_tokens;   /* GQA_DECODE_TILE: keys per wave tile, 0 = by head_dim and cache type; 16, 32 or 64
                          (ignored where a tile would exceed 16 KB of K+V per wave) */
    int double_buffer; /* GQA_DECODE_DBUF=1: two register tiles per wave (A/B variant); 0 (default): one */
    int pv_mode;       /* GQA_DECODE_PV=f32 -> 0: fp32-MFMA PV (A/B variant); 1 (default): bf16 MFMA, P hi+lo */
    int streaming;     /* GQA_DECODE_NT=0 -> 0: default cache policy; 1 (default): non-temporal K/V loads */
    int partition;     /* GQA_DECODE_PARTITION=fixed|even|prop -> 1|2|3; 0 (default): by shape.
                          prop (an A/B variant): every (sequence, kv head) of n tiles cut into
                          ceil(n / L) equal splits, L = ceil(all tiles / shares), decided on the
                          device from seq_lens -- one piece per workgroup, up to one more
                          workgroup per segment than shares; the combine kernel folds them */
    int shares;        /* GQA_DECODE_SHARES: even-share workgroups; 0 (default): two per CU for batches
                          (one per CU for long contiguous segments), one per CU for one sequence */
    int split_keys;    /* GQA_DECODE_SPLIT_KEYS: most keys per fixed split; 0 (default): 2048 */
    int piece_cost;    /* GQA_DECODE_PIECE_COST: tiles a piece's start and fold are worth in the even
                          partition, 0..1024; default 4 */
    int halve_long;    /* GQA_DECODE_HALVE_LONG=0 -> 0: keep two shares per CU for long contiguous bf16
                          segments; 1 (default): one per CU */
    int combine;       /* GQA_DECODE_COMBINE=tree -> 1: always the tree combine; 0 (default): by plan */
    int combine_cols;  /* GQA_DECODE_COMBINE_COLS: tree-combine columns per workgroup, 2, 4, 8 or 16;
                          0 (default): by grid size */
    int num_splits;    /* GQA_DECODE_SPLITS: splits used when a call passes num_splits = 0;
                          0 (default): the heuristic */
    int fold;          /* GQA_DECODE_FOLD=kernel|fused -> 1|2: fold the partials in a combine kernel (two
                          launches), or in the split kernel itself (one launch: the workgroup that writes
                          the last partial of a group, as counted by an arrival ticket in the workspace
                          header, folds the group -- every piece of a segment in the even partition, a
                          node of a fold tree over fixed splits -- in a fixed order, so results stay
                          bit-exact from run to run); 0 (default): the combine kernel, except for fixed
                          splits whose fold is one node of at most 16 partials, 16 KB in all, per
                          (sequence, kv head), which the split kernel folds (measured faster there
                          only) */
    int qk_mode;       /* GQA_DECODE_QK=valu -> 1: QK^T on the vector ALU (v_dot2c_f32_bf16 over each lane's
                          quarter of the head dims, two lane swaps, an LDS transpose) where the plan allows
                          it (bf16 cache and PV, one register tile, head_dim 128 or 256, 16-key tiles); an
                          A/B variant.  0 (default): bf16 MFMA */
} gqa_tuning_t;

/* The tuning calls use from now on (a copy). */
void gqa_decode_get_tuning(gqa_tuning_t *tuning);

/* Replace the tuning; GQA_ERR_NULL for NULL, GQA_ERR_SHAPE (nothing changed)
 * when a field is outside the range documented above. */
gqa_status_t gqa_decode_set_tuning(const gqa_tuning_t *tuning);

/*
 * The split plan for a call (the split-count rule of the AstrAI csrc commit
 * log: fill the device, bounded by the tile count).  max_seq_len is the cache
 * capacity (contiguous S_max, or max_pages * page_size when paged);
 * page_size = 0 means a contiguous cache.  num_splits = 0 picks the layout
 * from the shapes and cu_count: one sequence takes fixed splits (about one
 * workgroup per CU); a batch takes even shares (the concatenated tiles of all
 * sequences cut into equal parts on the device, from seq_lens), unless its
 * splits of one 16-key tile per wave take at most four workgroups per CU, in
 * which case it takes those fixed splits; a short cache may take a single
 * direct split.  num_splits > 0 forces that many fixed splits per (sequence,
 * kv head) (clamped to the tile count).  Pure host code: needs no GPU.
 */
gqa_status_t gqa_decode_plan(int B, int Hq, int Hkv, int head_dim, int max_seq_len, int page_size,
                             int num_splits, int cu_count, gqa_plan_t *plan);

/*
 * Workspace bytes gqa_decode / gqa_paged_decode need for the same arguments
 * on the current device.  With num_splits = 0 this queries the current
 * device's CU count; returns SIZE_MAX if the arguments are invalid or the
 * device cannot be queried.
 */
size_t gqa_decode_workspace_bytes(int B, int Hq, int Hkv, int head_dim, int max_seq_len,
                                  int page_size, int num_splits);

/*
 * Contiguous cache.
 *   q        bf16 [B][Hq][head_dim]
 *   k_cache  bf16 [B][Hkv][S_max][head_dim]
 *   v_cache  bf16 [B][Hkv][S_max][head_dim]
 *   seq_lens int32 [B], each in [0, S_max]
 *   out      fp32 [B][Hq][head_dim]  (written)
 *   The whole [S_max] extent of every (b, kv head) must be readable: rows at
 *   or past seq_lens[b] may be loaded (one tile's worth, before the length is
 *   known) but never contribute to the result, whatever they hold (NaN too).
 *   workspace: at least gqa_decode_workspace_bytes(B, Hq, Hkv, head_dim,
 *              S_max, 0, num_splits) bytes; may be NULL when that is 0.
 *              Its first 16384 bytes hold the arrival counters of the
 *              in-kernel fold (gqa_tuning_t.fold): they must be ZERO before
 *              the workspace is first used (zero the whole buffer once after
 *              allocating it, e.g. hipMemset, outside any graph capture), and
 *              every call leaves them zero again.  The rest needs no
 *              initialisation: it carries one call's partials from the split
 *              workgroups to the fold.  Calls that share a workspace must not
 *              run concurrently (one stream orders them).
 *   num_splits: 0 = heuristic, > 0 = forced.
 */
gqa_status_t gqa_decode(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim, int S_max,
                        float scale, float *out, void *workspace, size_t workspace_bytes,
                        int num_splits, hipStream_t stream);

/*
 * Paged cache (AstrAI csrc/tests commit log, the paged decode bullets: one
 * page-table lookup per tile, a tile never straddling a page).
 *   k_pool, v_pool bf16 [num_pages][Hkv][page_size][head_dim]
 *   page_table     int32 [B][max_pages]; token t of sequence b is row
 *                  t % page_size of page page_table[b][t / page_size]
 *   page_size      a positive multiple of 16
 *   seq_lens[b] <= max_pages * page_size
 *   Other arguments as gqa_decode; the workspace size uses
 *   max_seq_len = max_pages * page_size and page_size.
 */
gqa_status_t gqa_paged_decode(const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *seq_lens, const int32_t *page_table, int B, int Hq,
                              int Hkv, int head_dim, int page_size, int num_pages, int max_pages,
                              float scale, float *out, void *workspace, size_t workspace_bytes,
                              int num_splits, hipStream_t stream);

/*
 * The two steps of a call, for callers that schedule them separately (the
 * split-KV partial kernel, then the combine kernel).  gqa_decode_partials /
 * gqa_paged_decode_partials take exactly the arguments of gqa_decode /
 * gqa_paged_decode and launch only the split kernel: it leaves the
 * unnormalised (m, l, acc) partials in `workspace` (when the plan is direct
 * it writes `out` instead).  gqa_decode_combine then folds those partials
 * into `out` (it launches nothing for a direct plan); its seq_lens, shape
 * arguments, num_splits and the tuning (gqa_tuning_t) must be those of the
 * partials call, so that both compute the same plan (max_seq_len = S_max and
 * page_size = 0 for a contiguous cache).  Running the two on one stream gives bit-for-bit the
 * result of the one-call entry point.
 */
gqa_status_t gqa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim,
                                 int S_max, float scale, float *out, void *workspace,
                                 size_t workspace_bytes, int num_splits, hipStream_t stream);

gqa_status_t gqa_paged_decode_partials(const void *q, const void *k_pool, const void *v_pool,
                                       const int32_t *seq_lens, const int32_t *page_table, int B,
                                       int Hq, int Hkv, int head_dim, int page_size, int num_pages,
                                       int max_pages, float scale, float *out, void *workspace,
                                       size_t workspace_bytes, int num_splits, hipStream_t stream);

gqa_status_t gqa_decode_combine(const void *workspace, size_t workspace_bytes,
                                const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim,
                                int max_seq_len, int page_size, int num_splits, float *out,
                                hipStream_t stream);

/*
 * FP8 (E4M3) KV cache: the quantized pool of sparkinfer PR #874, section
 * "Cost and fallbacks" (an int8 pool dequantised before use), in the format
 * native to gfx950.  k_cache / v_cache (or the pools) hold OCP FP8 E4M3 bytes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals at
 * exponent 0; 0x7F / 0xFF are NaN) in the layouts of gqa_decode /
 * gqa_paged_decode with one byte per element, 16-byte aligned.  An element's
 * value is k_scale (resp. v_scale) times its E4M3 value; both scales must be
 * finite.  Every E4M3 value is exactly a bf16 value, so K and V enter the
 * same bf16 MFMA contractions as the bf16 cache; k_scale is folded into the
 * softmax scale and v_scale into the partials.  All other arguments, the
 * workspace (gqa_decode_workspace_bytes with the same shapes) and the
 * behaviour are those of gqa_decode / gqa_paged_decode.
 */
gqa_status_t gqa_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim,
                            int S_max, float scale, float k_scale, float v_scale, float *out,
                            void *workspace, size_t workspace_bytes, int num_splits,
                            hipStream_t stream);

gqa_status_t gqa_paged_decode_fp8(const void *q, const void *k_pool, const void *v_pool,
                                  const int32_t *seq_lens, const int32_t *page_table, int B, int Hq,
                                  int Hkv, int head_dim, int page_size, int num_pages, int max_pages,
                                  float scale, float k_scale, float v_scale, float *out,
                                  void *workspace, size_t workspace_bytes, int num_splits,
                                  hipStream_t stream);

/* The split kernel of gqa_decode_fp8 / gqa_paged_decode_fp8 alone (see the
 * *_partials entry points above); gqa_decode_combine_fp8 folds their partials. */
gqa_status_t gqa_decode_fp8_partials(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim,
                                     int S_max, float scale, float k_scale, float v_scale, float *out,
                                     void *workspace, size_t workspace_bytes, int num_splits,
                                     hipStream_t stream);

gqa_status_t gqa_paged_decode_fp8_partials(const void *q, const void *k_pool, const void *v_pool,
                                           const int32_t *seq_lens, const int32_t *page_table, int B,
                                           int Hq, int Hkv, int head_dim, int page_size,
                                           int num_pages, int max_pages, float scale,
                                           float k_scale, float v_scale, float *out,
                                           void *workspace, size_t workspace_bytes,
                                           int num_splits, hipStream_t stream);

/*
 * The plan of a call over an E4M3 cache (gqa_decode_plan's arguments and
 * rules), and the combine of gqa_decode_fp8_partials /
 * gqa_paged_decode_fp8_partials (gqa_decode_combine's arguments and rules).
 * A paged E4M3 cache at head_dim 128 takes 32-key tiles where bf16 takes 16,
 * so that a wave still reads 4 KB of K and of V in one piece of a page
 * (except small jobs, whose one-tile-per-wave splits take 16 for both); the
 * plan therefore depends on the element type, and the combine must recompute
 * the plan of the partials call.  The workspace a bf16 call of the same
 * shapes needs (gqa_decode_workspace_bytes) is always enough: longer tiles
 * never give more shares or splits.
 */
gqa_status_t gqa_decode_plan_fp8(int B, int Hq, int Hkv, int head_dim, int max_seq_len, int page_size,
                                 int num_splits, int cu_count, gqa_plan_t *plan);

gqa_status_t gqa_decode_combine_fp8(const void *workspace, size_t workspace_bytes,
                                    const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim,
                                    int max_seq_len, int page_size, int num_splits, float *out,
                                    hipStream_t stream);

/*
 * Multi-query decode (verification of M drafted tokens in speculative
 * decoding: the drafted block of the sparkinfer PR #874 speculative-decode
 * report; causal masking as in the prefill kernel of the AstrAI csrc commit
 * log).  Each sequence carries M query tokens, its last M positions, whose
 * keys and values are already in the cache: query i (0-based) attends to
 * keys 0 .. seq_lens[b] - M + i.
 *   q   bf16 [B][M][Hq][head_dim];  out fp32 [B][M][Hq][head_dim]
 *   M >= 1 and M * (Hq / Hkv) <= 16 (the M*G query rows of a kv head share
 *   every K/V byte; GQA_ERR_UNSUPPORTED otherwise).  A row with
 *   seq_lens[b] - M + i + 1 <= 0 is zero.
 *   workspace: gqa_decode_workspace_bytes(B, M * Hq, Hkv, head_dim, ...).
 * Everything else as gqa_decode / gqa_paged_decode (M = 1 is gqa_decode).
 */
gqa_status_t gqa_decode_mq(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, int B, int M, int Hq, int Hkv, int head_dim,
                           int S_max, float scale, float *out, void *workspace,
                           size_t workspace_bytes, int num_splits, hipStream_t stream);

gqa_status_t gqa_paged_decode_mq(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *seq_lens, const int32_t *page_table, int B, int M,
                                 int Hq, int Hkv, int head_dim, int page_size, int num_pages,
                                 int max_pages, float scale, float *out, void *workspace,
                                 size_t workspace_bytes, int num_splits, hipStream_t stream);

/*
 * gqa_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the partials live in a static device array of the
 * library, 4 MiB per GPU (4194304 bytes, held until the process ends), whose
 * address is looked up on the first call on each device.  The call allocates
 * nothing; the caller passes inputs and `out` as for gqa_decode (same
 * arguments without workspace / workspace_bytes, same results bit for bit).
 * A call whose plan needs more than 4 MiB of scratch
 * (gqa_decode_workspace_bytes) launches nothing and returns GQA_ERR_TOO_LARGE;
 * a batch of 16 sequences x 4 kv heads x 16384 keys at head_dim 128 needs
 * ~2.4 MB, a GQA-6 head_dim-256 layer of 4096 keys ~1.6 MB.  Every call on a GPU
 * shares that GPU's array and its contents: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race.
 */
gqa_status_t gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *seq_lens, int B, int Hq, int Hkv, int head_dim,
                                int S_max, float scale, float *out, int num_splits,
                                hipStream_t stream);

/* Static, human-readable text for a status code. */
const char *gqa_status_string(gqa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
