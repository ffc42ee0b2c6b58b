/*
 * dstopk.h -- DeepSelect row-wise top-k selection for AMD Instinct MI355X (gfx950).
 *
 * The method is DeepSelect as given in the DeepSelect design note ("Algorithm",
 * DeepSelectTopk pseudocode): keep a threshold T; read the row once, in blocks of B
 * elements taken in a random order that does not depend on the data; append the
 * elements that beat T to an on-chip candidate buffer; when the buffer holds at least
 * k + B2 entries, reduce it to the k best with a radix select and raise T to the
 * smallest of them; after the last block, one more radix select gives the answer.
 * Long rows can be cut into slices that run the method independently; a merge step
 * then selects the k best of the slices' survivors (the cluster split of the design
 * note's "Implementation" section, here through a device workspace).
 *
 * Result contract (the plain definition the method reaches exactly):
 *   for every row r, the k largest elements of x[r, 0..N) under the total order
 *   "larger value first; +0 before -0; then smaller index first", written in that
 *   order. Values are the input's own bit patterns; indices are int32, relative to the
 *   row. The result does not depend on `seed`, the block size or the slicing.
 *
 * Conventions for every entry point:
 *   - x, out_vals, out_idx, workspace and stats are DEVICE pointers (HIP).
 *   - stream is a hipStream_t passed as void*; NULL is the default stream.
 *   - All work is enqueued on `stream`; calls are asynchronous and never synchronise.
 *   - Arguments are validated on the host before anything is enqueued; an invalid call
 *     returns a negative status and enqueues nothing.
 *   - Precondition: x holds no NaN (the output is unspecified otherwise); +-inf and
 *     +-0 are allowed.
 *   - No entry point keeps a pointer after it returns.
 */
#ifndef DSTOPK_H
#define DSTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define DS_BF16 0 /* bfloat16, 2 bytes, the Lightning Indexer scores */
#define DS_FP32 1 /* float32, 4 bytes, the sampler logits */

/* status codes */
#define DS_OK 0
#define DS_ERR_INVALID_ARG (-1) /* bad sizes, k, pointers or dtype */
#define DS_ERR_UNSUPPORTED (-2) /* a forced configuration this build has no kernel for */
#define DS_ERR_ALIGNMENT (-3)   /* x or row_stride*elem_bytes not a multiple of 16 bytes */
#define DS_ERR_WORKSPACE (-4)   /* workspace missing or smaller than ds_topk_workspace_size */
#define DS_ERR_LAUNCH (-5)      /* the HIP runtime refused a launch or an allocation */
#define DS_ERR_DEVICE (-6)      /* no usable gfx950 device, or a device query failed */

/* The largest supported k: the DeepSelect library accepts top-k of at most 4096 and no more
 * (TileLang tutorial chapter 37, "DeepSelect top-k", section 1.2, the constraint matrix). */
#define DS_MAX_K 4096

/*
 * Launch configuration. Zero in any field means "choose automatically".
 *   block   B: elements per block; a multiple of 512 (bf16) or 256 (fp32) equal to
 *              waves * chunks_per_wave * that chunk size for one of the built kernels.
 *   slack   B2: the buffer is compacted when it holds >= k + B2 entries (B2 >= 1).
 *   slices  S: workgroups per row (the split-row path when > 1).
 *   waves   64-lane waves per workgroup.
 *   presample  the threshold before the first compaction: DS_PRESAMPLE_OFF starts from
 *              "accept everything" as the design note does, so the first block fills the
 *              buffer; DS_PRESAMPLE_ON starts from a lower bound of the first block's k-th
 *              largest element (each wave takes the ceil(k/waves)-th largest of its lanes'
 *              maxima, and the bound is the smallest of those, so at least k elements of
 *              the block reach it), and the block only appends the elements that reach it.
 *              ON needs k <= 64 * waves and a whole first block; otherwise the plan falls
 *              back to OFF. Zero (auto) means ON. The result is the same either way.
 *              The lanes' maxima are taken over every whole block among the first `depth`
 *              blocks of the order (all of them are requested at the start).
 *   order_group  G in {1, 2, 4}: the random order is drawn over groups of G consecutive
 *              blocks, which are read in turn (G = 1 is the design note's order of single
 *              blocks; larger G keeps consecutive loads in flight, measured faster on
 *              MI355X). Zero (auto) means 2 when a slice has at least 8 blocks, else 1.
 *              The result is the same for every G.
 *   merge      the merge step of split rows (slices > 1). DS_MERGE_LISTS: every slice
 *              writes its k survivors sorted, and the lists are merged in levels: each
 *              level merges groups of up to 16 consecutive lists (as many as fit in 128 KiB
 *              of LDS at 8 bytes an entry) into one sorted list of the group's k best, one
 *              workgroup per list placing its entries by binary searches in the group's
 *              other lists; the plan takes the fewest levels and the smallest equal group
 *              sizes that reach one list. DS_MERGE_SELECT: one workgroup per row runs
 *              DeepSelect again over the row's slices * k survivors. Zero (auto) means
 *              LISTS. The plan reports the merge used (0 when slices == 1).
 */
#define DS_PRESAMPLE_AUTO 0
#define DS_PRESAMPLE_OFF 1
#define DS_PRESAMPLE_ON 2
#define DS_MERGE_AUTO 0
#define DS_MERGE_LISTS 1
#define DS_MERGE_SELECT 2
/*
 *   schedule   when the buffer is checked. DS_SCHEDULE_LOCKSTEP is the design note's schedule
 *              ("Algorithm", the DeepSelectTopk pseudocode): every wave of the workgroup
 *              filters its share of a block, a workgroup barrier follows, and then the buffer
 *              is compacted if it holds at least k + B2 entries. DS_SCHEDULE_FREE drops the
 *              barrier after every block: each wave streams
 *              its shares on its own, reserves buffer space with one atomic and checks the
 *              length itself after every share; a wave that sees k + B2 or more stops at a
 *              barrier and the waves compact together. A wave appends at most one more share
 *              after the length crosses k + B2, so the buffer bound k + B2 + B of the design
 *              note's notes still holds. The result is the same for both; only the counters
 *              (which elements were appended with which threshold) differ. Zero (auto): FREE,
 *              or LOCKSTEP when B2 < B / 2 (the buffer then fills within a block, and the
 *              once-per-block check measured faster).
 */
#define DS_SCHEDULE_AUTO 0
#define DS_SCHEDULE_FREE 1
#define DS_SCHEDULE_LOCKSTEP 2

typedef struct ds_config {
  int32_t block;
  int32_t slack;
  int32_t slices;
  int32_t waves;
  int32_t presample;
  int32_t order_group;
  int32_t merge;
  int32_t schedule;
  int32_t depth; /* output only (ds_topk_plan): blocks in flight per wave; zero on input */
  int32_t output;
  int32_t warmup;
  int32_t share;
} ds_config;
/*
 *   output     flags for the outputs' form (zero: sorted, int32 indices).
 *              DS_OUTPUT_UNSORTED: each row's k outputs are its top k in an unspecified
 *              order (tutorial chapter 37, sections 5.1 and 5.2(4): the Ascend kernel leaves
 *              its output unsorted and sorts only the k results, at the end, when asked).
 *              The single-slice path then skips the final sort (the survivors of the final
 *              compaction are written as they stand) and so does the merge kernel
 *              (DS_MERGE_SELECT); the list merge still writes sorted rows.
 *              DS_OUTPUT_INDEX_INT64: out_idx is [rows, k] int64 (TileKernels chapter 33,
 *              section 4.7: the gate's indices are int64, converted exactly from int32).
 */
#define DS_OUTPUT_UNSORTED 1
#define DS_OUTPUT_INDEX_INT64 2
/*
 *   warmup     w >= 0 blocks of warm-up window (tutorial chapter 37, section 5.2(1): the
 *              first shuffled pages are radix-selected to set the threshold before the
 *              steady stream; the CUDA side's init window does the same). The first w blocks
 *              of each slice's order are appended unfiltered and checked after every block;
 *              after the w-th, a buffer of more than k entries is compacted, so T becomes
 *              the k-th best of the window. Then the schedule continues as planned. A
 *              window turns the presampled start off. Zero (default): no window.
 *   share      DS_SHARE_ON: the slices of a split row share a threshold (design note,
 *              "Implementation", cluster paragraph: the parts of a row work toward one
 *              top-k; tutorial chapter 37, section 4.7). Each slice publishes its threshold
 *              (the presampled T0 and every compaction's k-th entry) to a per-row word with
 *              an atomic maximum and filters with the larger of its own and the row's; every
 *              published value ranks at or below the row's k-th element, so the result is
 *              unchanged and only the work shrinks (counters become timing-dependent). The
 *              row words take rows * 8 bytes (rounded up to 16) at the start of the workspace
 *              and are zeroed by a small kernel before each select launch. Zero (auto): ON
 *              for split rows without the presampled start (large k), else OFF. The plan
 *              reports ON, or OFF for split rows (AUTO when the plan has one slice).
 */
#define DS_SHARE_AUTO 0
#define DS_SHARE_OFF 1
#define DS_SHARE_ON 2

/*
 * Per-(row, slice) counters of one run, filled when ds_topk_ex gets a stats pointer.
 * Names follow the design note's analysis section ("Expected Upper Bound on the Total
 * Elements Processed by RadixSelectTopK": A, R, W). Under DS_SCHEDULE_LOCKSTEP every
 * counter is a function of (x, k, B, B2, seed, slicing); under DS_SCHEDULE_FREE reads,
 * index_sum and monotone are, while A, R, W and max_len depend on how the waves interleave
 * (W = A + k*R, R*B2 <= A and max_len <= k + B2 + B - 1 hold for both).
 */
typedef struct ds_stats {
  uint64_t appended;    /* A: elements appended to the candidate buffer */
  uint64_t compactions; /* R: in-loop radix-select compactions */
  uint64_t work;        /* W: summed input sizes of all compactions, the final one included */
  uint64_t max_len;     /* largest buffer length after a block's appends */
  uint64_t reads;       /* elements read from x */
  uint64_t index_sum;   /* sum of the row indices of the elements read */
  uint64_t monotone;    /* 1 if every new threshold ranked at or below the previous one */
  uint64_t slice_lo;    /* first row index of the slice */
  uint64_t slice_len;   /* elements in the slice */
  uint64_t block;       /* B used */
  uint64_t slack;       /* B2 used */
  uint64_t t_total_ns;  /* workgroup wall time (device real-time clock, 10 ns ticks) */
  uint64_t t_compact_ns; /* time in in-loop compactions */
  uint64_t t_sync_ns;   /* time in the per-block barrier */
  uint64_t t_final_ns;  /* time in the final compaction and output */
  uint64_t passes;      /* histogram passes of all compactions, the final one included */
} ds_stats;

/*
 * ds_topk -- top-k of every row (DeepSelect design note, "Algorithm": DeepSelectTopk, whose
 * final RadixSelectTopK returns exactly the k largest; ties go to the smaller index, the
 * convention of TileLang tutorial chapter 33's top-k gate reference).
 *   x          device, rows x row_stride elements of `dtype`; row r starts at
 *              x + r*row_stride elements. 16-byte aligned; row_stride*elem_bytes a
 *              multiple of 16 (DS_ERR_ALIGNMENT otherwise): the scan reads 16-byte vectors.
 *              The DeepSelect library has its own row-stride alignment contract (tutorial
 *              chapter 37, section 1.2); 16 bytes is this build's.
 *   rows       >= 0; rows == 0 returns DS_OK and enqueues nothing.
 *   n          elements per row, 1 <= n <= 2^31 - 1; row_stride >= n.
 *   k          1 <= k <= min(DS_MAX_K, n) (the pseudocode's "require 1 <= k <= N").
 *   dtype      DS_BF16 (Lightning Indexer scores) or DS_FP32 (sampler logits): the two
 *              input types of tutorial chapter 37, sections 1.1-1.2.
 *   seed       picks the block order only; it never changes the result (design note: the
 *              permutation is independent of x and only the cost is random).
 *   out_vals   device [rows, k] of `dtype` (bit patterns of the selected elements), or NULL.
 *   out_idx    device [rows, k] int32, or NULL (values only). Not both NULL.
 *   stream     hipStream_t as void*.
 * When the split path needs scratch memory, ds_topk takes it from a cache that holds one
 * buffer per (device, stream): calls on one stream share it (the stream orders them), calls
 * on different streams never do. A cached buffer is never freed before the library is
 * unloaded (when a stream needs more, its old buffer is kept aside), so a graph that
 * captured a call keeps a valid buffer. Growing the cache calls hipMalloc on the calling
 * thread; on a stream that is being captured it returns DS_ERR_WORKSPACE instead (capture
 * a ds_topk_ex call with its own workspace, or make one uncaptured call of the same size on
 * that stream first).
 */
int ds_topk(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, uint64_t seed,
            void* out_vals, int32_t* out_idx, void* stream);

/*
 * ds_topk_plan -- the configuration ds_topk / ds_topk_ex would use (cfg may force some
 * fields; NULL = all automatic). Writes it to *out. Host only, no device call except a
 * one-time query of the current device's compute-unit count. The parameters are the
 * design note's B and B2 ("Algorithm") and the cluster split's parts per row
 * ("Implementation", last paragraph).
 */
int ds_topk_plan(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, ds_config* out);

/*
 * ds_topk_workspace_size -- bytes of device workspace ds_topk_ex needs for this call
 * (0 when the plan has one slice per row). Writes it to *bytes. The workspace holds each
 * part's k survivors on their way to the merge, where the design note's cluster split
 * ("Implementation", last paragraph) sends them to the first block of the cluster.
 */
int ds_topk_workspace_size(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, size_t* bytes);

/*
 * ds_topk_ex -- ds_topk with a caller workspace, a forced configuration and counters
 * (the same method: design note, "Algorithm"; the counters of its "Expected Upper Bound"
 * section).
 *   workspace  device, >= ds_topk_workspace_size bytes, 16-byte aligned; may be NULL when
 *              that size is 0. Its contents on entry do not matter; it is overwritten.
 *              Calls that share a workspace must not overlap in time.
 *   lens       NULL, or device [rows] int32: ragged rows (tutorial chapter 37, section 5.2(1):
 *              the Ascend kernel takes each row's valid length; a DSA indexer query sees
 *              its own context length, section 1.1). Row r is its first
 *              min(max(lens[r], 0), n) elements; n (the longest row) sets the plan. When a
 *              row holds fewer than k elements, its outputs past them are padding: index -1
 *              and the value bit pattern of all ones (a NaN, never an input). The values are
 *              read on the device only.
 *   out_idx    as in ds_topk, or [rows, k] int64 when cfg->output has DS_OUTPUT_INDEX_INT64
 *              (8-byte aligned).
 *   cfg        NULL or fields to force (see ds_config).
 *   stats      NULL, or device [rows, slices] ds_stats filled by the select kernel.
 * Allocates nothing and never synchronises, so it can be captured in a graph.
 */
int ds_topk_ex(const void* x, const int32_t* lens, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype,
               uint64_t seed, void* out_vals, void* out_idx, void* workspace, size_t ws_bytes, const ds_config* cfg,
               ds_stats* stats, void* stream);

/*
 * ds_topk_slices / ds_topk_merge -- ds_topk_ex as its two launches (the per-part top-k and
 * the merge of the design note's cluster split, "Implementation", last paragraph), for callers that
 * want to time or overlap them separately. ds_topk_slices runs the select kernel: with one
 * slice per row it writes the final outputs; otherwise it writes every slice's k survivors
 * to the workspace (sorted, for the list merge) and ds_topk_merge reduces each row's
 * survivors to the sorted top-k (one launch per list-merge level, or one merge-kernel
 * launch; nothing when the plan has one slice). Both take the same arguments as
 * ds_topk_ex (merge ignores x, row_stride and stats) and must be given the same lens, rows,
 * n, k, dtype, seed, cfg and workspace; the pair then equals one ds_topk_ex call.
 */
int ds_topk_slices(const void* x, const int32_t* lens, int64_t rows, int64_t n, int64_t row_stride, int k,
                   int dtype, uint64_t seed, void* out_vals, void* out_idx, void* workspace, size_t ws_bytes,
                   const ds_config* cfg, ds_stats* stats, void* stream);
int ds_topk_merge(const int32_t* lens, int64_t rows, int64_t n, int k, int dtype, uint64_t seed, void* out_vals,
                  void* out_idx, void* workspace, size_t ws_bytes, const ds_config* cfg, void* stream);

/*
 * ds_topk_noalloc -- ds_topk for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, plan, kernels and result as ds_topk; the split rows' workspace is a
 * library-owned device array of DS_NOALLOC_SCRATCH_BYTES on each GPU (reserved when the
 * library's code is loaded on that GPU and held until the process ends) instead of the
 * per-stream cache, so no call allocates, frees or synchronises. A call whose plan needs
 * more workspace than that returns DS_ERR_WORKSPACE and enqueues nothing (use ds_topk_ex
 * with a workspace of ds_topk_workspace_size bytes). All calls on one GPU share the one
 * array, on every stream: calls that overlap in time on one GPU race and give wrong
 * results, so order them (one stream, or events). Nothing in the array needs to start at
 * any value; each call overwrites what it reads.
 */
#define DS_NOALLOC_SCRATCH_BYTES (8u << 20)
int ds_topk_noalloc(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, uint64_t seed,
                    void* out_vals, int32_t* out_idx, void* stream);

/*
 * ds_probe_read -- measurement aid, not part of top-k (tutorial chapter 37, section 6.1: the
 * method's measure is how close it comes to reading the input once; this is the plain read
 * of the same bytes): streams `bytes` (a multiple of
 * 16, 16-byte aligned) from src with the same 16-byte loads the scan uses and writes
 * one 32-bit word per workgroup to sink (device, >= ds_probe_sink_words(bytes) words).
 */
int ds_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);
int64_t ds_probe_sink_words(int64_t bytes);

/* ds_probe_copy -- measurement aid: a plain 16-byte-vector copy of `bytes` (multiple of 16),
 * whose known byte counts calibrate the HBM traffic counters. */
int ds_probe_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* ds_status_string -- a static, human-readable name for a status code (never NULL). */
const char* ds_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSTOPK_H */
