/*
 * adacomp.h -- C ABI of the AdaComp compressor for AMD Instinct MI355X (gfx950).
 *
 * AdaComp ("AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
 * page, definition paragraph and the Mechanism claim on local-bin soft
 * threshold and mean-g_max quantization, Algorithm 2) compresses each layer's
 * gradient dW against a residue carried from step to step:
 *
 *   G = residue + dW,  H = G + dW                       (float32, no contraction)
 *   bins of L_T consecutive elements; g_max(i) = max |G| over bin i
 *   transmit every element with |H| >= g_max(its bin) and G != 0
 *   s = mean of g_max over the layer's bins             (one scale per layer)
 *   G_q = sign(G) * s for transmitted elements
 *   residue <- G - G_q (transmitted), residue <- G (all others)
 *
 * The transmitted elements are packed as sparse-indexed ternary words, 8-bit
 * when L_T < 64 and 16-bit otherwise (Application claim, Table 2; Curated
 * Limitations), into a message whose length varies from step to step
 * (Limitation claim).  decode_accumulate sums several such messages, one per
 * learner of a data-parallel job, into a dense float32 gradient.
 *
 * Conventions common to every call:
 *   - Every pointer named residue, dW, out, msg, msgs[k] or ws is a DEVICE
 *     pointer on the device that was current when the plan was created; that
 *     device must be current at the call.  Pointers to plain structs and to
 *     the msgs array are HOST pointers.  The caller owns every buffer.
 *   - The flat float32 buffers (residue, dW, out) hold every layer of the
 *     segment table at its element offset; they must be 16-byte aligned and
 *     hold at least info.span elements (the end of the last layer rounded up
 *     to a multiple of 4).  Elements outside every segment may be read but
 *     are never written.
 *   - msg and ws must be 16-byte aligned and at least as large as the plan
 *     reports.  Buffers given to one call must not overlap.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream) and return once the work is enqueued.  Argument errors are
 *     detected on the host before anything is enqueued, and then nothing is
 *     written.  Results are deterministic: the same inputs give the same bits.
 *   - Return value: ADACOMP_OK (0) or a negative status; adacomp_status_str()
 *     names it.  No C++ exception crosses this interface.
 *
 * Message layout (all little-endian, every region 16-byte aligned, padding
 * bytes zero; w = 8 if L_T < 64 else 16):
 *   header, 32 bytes: u32 magic 0x43414441 ("ADAC"), u16 version 1, u16 0,
 *     u32 nseg, u32 plan_hash, u64 total_bytes, u64 total_survivors;
 *   directory at byte 32: nseg x 16 bytes {f32 s, u32 nsurv, u64 entries_offset};
 *   count regions, one per segment in table order, at positions fixed by the
 *     plan: B words of w bits, the number of transmitted elements per bin;
 *   entry regions, one per segment in table order, packed after the count
 *     regions: nsurv words of w bits, bin-major with ascending in-bin index,
 *     each word = sign << (w-1) | in_bin_index, sign = 1 iff G < 0.
 */
#ifndef ADACOMP_H
#define ADACOMP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ADACOMP_OK 0
#define ADACOMP_ERR_INVALID_ARGUMENT (-1) /* null pointer, empty table, numel 0, unknown flags, wrong device, aliasing */
#define ADACOMP_ERR_UNSUPPORTED_BIN (-2)  /* L_T = 0 or L_T > 32768 (a 16-bit word holds a 15-bit index) */
#define ADACOMP_ERR_MISALIGNED (-3)       /* segment offset not a multiple of 4, or a buffer not 16-byte aligned */
#define ADACOMP_ERR_OVERLAP (-4)          /* two segments share an element */
#define ADACOMP_ERR_CAPACITY (-5)         /* a buffer is smaller than the plan requires */
#define ADACOMP_ERR_HIP (-6)              /* a HIP runtime call or kernel launch failed */
#define ADACOMP_ERR_TOO_LARGE (-7)        /* numel >= 2^32 in one segment, or the table exceeds launch limits */
#define ADACOMP_ERR_SCRATCH_LIMIT (-8)    /* adacomp_compress_noalloc: the plan's workspace exceeds its scratch */

#define ADACOMP_MAX_BIN_LEN 32768u

/* Segment flag: hard Local Selection (LS) instead of AdaComp's soft threshold.
 * The baseline the same page's Mechanism claim "self-adjusting sparsity
 * prevents residual explosion" (Figures 4-6) contrasts AdaComp with: per bin
 * only the first element (lowest index) whose |G| equals the bin maximum is
 * transmitted, none when the maximum is 0; s, the residue update and the
 * message format are those of AdaComp. */
#define ADACOMP_SEG_LS 1u
#define ADACOMP_MAX_MESSAGES 256u         /* most messages one decode_accumulate call sums */

/* One layer: numel consecutive elements of the flat buffers starting at
 * element `offset` (a multiple of 4), compressed with bins of bin_len = L_T
 * elements over its flattened storage order.  flags: 0 (AdaComp) or
 * ADACOMP_SEG_LS. */
typedef struct adacomp_segment {
    uint64_t offset;
    uint64_t numel;
    uint32_t bin_len;
    uint32_t flags;
} adacomp_segment;

/* Sizes a caller needs to allocate buffers for a segment table. */
typedef struct adacomp_plan_info {
    uint32_t nseg;
    uint32_t plan_hash;                 /* FNV-1a 32 of the table, as in message headers */
    uint64_t total_numel;               /* sum of numel */
    uint64_t span;                      /* max(offset + numel) rounded up to a multiple of 4:
                                           the minimum length of residue, dW and out */
    uint64_t total_bins;                /* sum over segments of ceil(numel / bin_len) */
    uint64_t ntiles;                    /* work tiles (whole bins of one segment each) */
    uint64_t header_bytes;              /* 32 + 16*nseg: read this much to learn a message's size */
    uint64_t message_capacity;          /* largest possible message: every element transmitted */
    uint64_t compress_workspace_bytes;
    uint64_t decode_workspace_bytes_per_message;
    uint64_t decode_workspace_bytes_fixed; /* decode ws for K messages = fixed + K * per_message */
    uint64_t compress_launches;         /* kernel launches of one adacomp_compress call */
} adacomp_plan_info;

typedef struct adacomp_plan adacomp_plan;   /* opaque, immutable once created */
typedef struct adacomp_timer adacomp_timer; /* opaque per-kernel device timer */

/* Host-only: validate a segment table and report the sizes its plan would
 * have.  Touches no GPU.  Returns a status; fills *info on success. */
int adacomp_plan_query(const adacomp_segment* segs, uint32_t nseg, adacomp_plan_info* info);

/* Validate the table, build the work tiles and copy the small tile tables to
 * the current device.  The plan owns that device memory until
 * adacomp_plan_destroy.  An immutable plan may be used from several streams
 * at once (with separate buffers).
 *
 * Compress is one tile-pass launch per tile shape used (bins up to 2045,
 * up to 4093, longer), then the finish: survivor offsets, s, header and
 * directory, entry words and residue of the sent elements.  For a small
 * table -- span <= ADACOMP_SMALL_TABLE_MAX_SPAN elements and at most
 * ADACOMP_SMALL_TABLE_MAX_SEGMENTS segments -- the finish is one launch
 * whose every workgroup holds the table's tile counts in LDS.  Otherwise, for
 * a table of at most ADACOMP_SMALL_TABLE_MAX_SEGMENTS segments and at most
 * ADACOMP_CHUNK_FINISH_MAX_TILES tiles (info.ntiles), it is two: the chunk
 * scan, then one kernel whose every workgroup computes s and the entry
 * regions from the chunk sums in LDS and encodes its share.  Any other table
 * takes three (chunk scan, finalize, encode).  info.compress_launches reports
 * the total.  Every path writes the same bytes.  plan_query reports the sizes
 * of a plan made with no flags. */
#define ADACOMP_SMALL_TABLE_MAX_SPAN (1u << 21)
#define ADACOMP_SMALL_TABLE_MAX_SEGMENTS 256u
#define ADACOMP_CHUNK_FINISH_MAX_TILES (1u << 20)
int adacomp_plan_create(const adacomp_segment* segs, uint32_t nseg, adacomp_plan** plan);

/* Plan flags (adacomp_plan_create_ex).
 * SEPARATE_FINISH: finish with the three kernels whatever the table.
 * SINGLE_LAUNCH: compress a small table whose bins are all <= 4093 in one
 *   launch: the workgroup that finishes its tile last completes the message
 *   alone.  Correct, but slower on MI355X than the default (the release of
 *   every tile and one CU's scattered stores cost more than the launches it
 *   saves); built for comparison.  Other tables ignore it.
 * The two flags are exclusive.
 * DECODE_RECORDS: plain sums (adacomp_decode_accumulate with accumulate = 0)
 *   of at most 16 messages over bins of at most 4093 elements always take the
 *   entry-record decode (a per-tile record pass, then tiles that read their
 *   count and entry words in one round trip).  By default only tables of at
 *   least 65536 such tiles, all of 16-bit words, take it; smaller tables and
 *   8-bit words measured faster without it.  Combines with either flag above. */
#define ADACOMP_PLAN_SEPARATE_FINISH 1u
#define ADACOMP_PLAN_SINGLE_LAUNCH 2u
#define ADACOMP_PLAN_DECODE_RECORDS 4u
/* adacomp_plan_create with plan flags (0, or an OR of the above with at most
 * one of SEPARATE_FINISH and SINGLE_LAUNCH; any other value is
 * ADACOMP_ERR_INVALID_ARGUMENT). */
int adacomp_plan_create_ex(const adacomp_segment* segs, uint32_t nseg, uint32_t plan_flags,
                           adacomp_plan** plan);
int adacomp_plan_destroy(adacomp_plan* plan);
int adacomp_plan_get_info(const adacomp_plan* plan, adacomp_plan_info* info);

/* One AdaComp compression step over every segment (the definition above).
 *   residue  [span] float32, read and updated in place.
 *   dW       [span] float32, read only.
 *   n_elems  elements in residue and in dW (>= info.span).
 *   msg      message output, msg_bytes >= info.message_capacity.  Its length
 *            is the header's total_bytes (read it after the stream syncs).
 *   ws       workspace, ws_bytes >= info.compress_workspace_bytes; no
 *            initial contents required, contents undefined afterwards, except
 *            that with ADACOMP_PLAN_SINGLE_LAUNCH its first 8 bytes hold a
 *            ticket counter: a 48-bit tag above a 16-bit count, left with
 *            count 0.  Any other initial value is accepted; only the tag with
 *            a nonzero count (a call stopped part way) would miscount.
 *   bin_max_out  nullable device float32[total_bins]: every g_max, segments
 *            in table order, bins in order (a testing aid).
 * Determinism: s is the bin maxima summed in float64 in a fixed order, divided
 * by B in float64 and rounded once to float32; everything else is exact. */
int adacomp_compress(const adacomp_plan* plan, float* residue, const float* dW,
                     uint64_t n_elems, void* msg, uint64_t msg_bytes, void* ws,
                     uint64_t ws_bytes, float* bin_max_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one
 * compression step exactly as adacomp_compress, with the workspace taken
 * from a scratch array the library holds on each GPU it runs on, from the
 * first call on that GPU until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or other allocating routine).
 *   Arguments as for adacomp_compress, without ws and ws_bytes; the current
 *   device must be the plan's.
 *   The plan's info.compress_workspace_bytes must be at most
 *   ADACOMP_NOALLOC_SCRATCH_BYTES (128 MiB: tables of up to about 33 million
 *   elements); larger plans return ADACOMP_ERR_SCRATCH_LIMIT before any work.
 *   Every call on one GPU shares that GPU's scratch and it keeps the last
 *   call's contents (compress needs no initial contents): calls that may
 *   overlap on one GPU -- on different streams, or from different threads
 *   without ordering -- race and must not be issued. */
#define ADACOMP_NOALLOC_SCRATCH_BYTES (128ull << 20)
int adacomp_compress_noalloc(const adacomp_plan* plan, float* residue, const float* dW,
                             uint64_t n_elems, void* msg, uint64_t msg_bytes, float* bin_max_out,
                             void* stream);

/* Sum K messages made by adacomp_compress with this same segment table into
 * out, in message order: for k = 0..K-1 and every element j message k
 * transmits, out[j] = out[j] + sign * s (float32, rounded each time).
 *   msgs        HOST array of K device pointers; 1 <= K <= ADACOMP_MAX_MESSAGES.
 *   out         [span] float32.  accumulate = 0: every element of every
 *               segment starts from +0; accumulate = 1: starts from out.
 *               An element no message transmits gets no addition.
 *   ws          ws_bytes >= fixed + K * per_message (see plan info).
 * Each msgs[k] must point to at least the header's total_bytes readable
 * bytes (at least 32).  A message is checked on the device before any entry
 * word is read, and is refused -- it contributes nothing, the other messages
 * are summed as if it were absent -- when its header does not match the plan
 * (magic, version, nseg, plan_hash; total_bytes a multiple of 16 between the
 * start of the entry regions and info.message_capacity), or when a segment's
 * directory entry disagrees with the count words (entry offset not 16-byte
 * aligned or before the entry regions; survivors more than the segment's
 * elements or unequal to the sum of its count words; a tile counting more
 * survivors than it has elements; the padded entry region past total_bytes).
 * Entry words whose in-bin index lies outside the bin are ignored.  The
 * number of refused messages is written as a uint32 at byte 0 of ws; the
 * call itself still returns ADACOMP_OK. */
int adacomp_decode_accumulate(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                              float* out, uint64_t n_elems, int accumulate, void* ws,
                              uint64_t ws_bytes, void* stream);

/* One step of SGD with momentum (no dampening, no Nesterov), the optimizer the
 * paper's abstract names for its training runs, taken on the summed messages:
 *   g = scale * sum (+ weight_decay * w when weight_decay != 0)
 *   m = momentum * m + g
 *   w = w - lr * m
 * each operation one float32 operation rounded to nearest. */
typedef struct adacomp_sgd {
    float lr;
    float momentum;
    float weight_decay;
    float scale;    /* e.g. 1/K to average the learners' gradients */
} adacomp_sgd;

/* Sum K messages exactly as adacomp_decode_accumulate with accumulate = 0 and
 * take one adacomp_sgd step on every element of every segment, without
 * writing the sum to memory (one dense pass instead of decode + optimizer).
 *   weights, momentum  [span] float32 each, updated in place; elements
 *               outside every segment are not written.
 *   sgd         HOST pointer to the step's parameters.
 *   ws          ws_bytes >= adacomp_decode_sgd_workspace_bytes(plan, K); plans
 *               with bins longer than 4093 elements need a dense scratch of
 *               4 * span bytes in it.
 * Messages are checked, refused and counted at byte 0 of ws as in
 * adacomp_decode_accumulate. */
int adacomp_decode_sgd(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                       float* weights, float* momentum, uint64_t n_elems, const adacomp_sgd* sgd,
                       void* ws, uint64_t ws_bytes, void* stream);
int adacomp_decode_sgd_workspace_bytes(const adacomp_plan* plan, uint32_t K, uint64_t* bytes);

/* One Adam step with bias-corrected moments (the other optimizer the paper's
 * abstract names), in its textbook form, each operation one float32
 * operation rounded to nearest (division and square root correctly rounded):
 *   g = scale * sum (+ weight_decay * w when weight_decay != 0)
 *   m = beta1 * m + (1 - beta1) * g;   v = beta2 * v + (1 - beta2) * (g * g)
 *   w = w - lr * ((m / c1) / (sqrt(v / c2) + eps))
 * c1 = 1 - beta1^step, c2 = 1 - beta2^step, each computed in double on the
 * host and rounded once to float; 1 - beta1 and 1 - beta2 are float
 * operations.  step >= 1 counts the calls made so far, this one included. */
typedef struct adacomp_adam {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    float scale;
    uint32_t step;
} adacomp_adam;

/* As adacomp_decode_sgd, with one Adam step on weights, m and v ([span]
 * float32 each, updated in place).  ws as for adacomp_decode_sgd
 * (adacomp_decode_sgd_workspace_bytes).  step = 0 is an invalid argument. */
int adacomp_decode_adam(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                        float* weights, float* m, float* v, uint64_t n_elems,
                        const adacomp_adam* adam, void* ws, uint64_t ws_bytes, void* stream);

/* Same calls with a timer: device time of each kernel stage is recorded with
 * HIP events on `stream` and summed in the timer.  timer may be NULL. */
int adacomp_compress_timed(const adacomp_plan* plan, float* residue, const float* dW,
                           uint64_t n_elems, void* msg, uint64_t msg_bytes, void* ws,
                           uint64_t ws_bytes, float* bin_max_out, void* stream,
                           adacomp_timer* timer);
int adacomp_decode_accumulate_timed(const adacomp_plan* plan, const void* const* msgs,
                                    uint32_t K, float* out, uint64_t n_elems, int accumulate,
                                    void* ws, uint64_t ws_bytes, void* stream,
                                    adacomp_timer* timer);
int adacomp_decode_sgd_timed(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                             float* weights, float* momentum, uint64_t n_elems,
                             const adacomp_sgd* sgd, void* ws, uint64_t ws_bytes, void* stream,
                             adacomp_timer* timer);
int adacomp_decode_adam_timed(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                              float* weights, float* m, float* v, uint64_t n_elems,
                              const adacomp_adam* adam, void* ws, uint64_t ws_bytes, void* stream,
                              adacomp_timer* timer);

/* Kernel stages a timer reports, in this order. */
#define ADACOMP_STAGE_TILE_PASS 0   /* dense pass: G, H, bin maxima, selection, counts */
#define ADACOMP_STAGE_CHUNK_SCAN 1  /* per-chunk survivor offsets and scale partial sums */
#define ADACOMP_STAGE_FINALIZE 2    /* s per segment, message header and directory (three-kernel finish) */
#define ADACOMP_STAGE_ENCODE 3      /* entry words and residue of transmitted elements */
#define ADACOMP_STAGE_DECODE_COUNT 4
#define ADACOMP_STAGE_DECODE_BASE 5
#define ADACOMP_STAGE_DECODE_APPLY 6
#define ADACOMP_STAGE_COMPRESS_CALL 7  /* a whole adacomp_compress call, gaps between kernels included
                                          (a small-table or two-kernel finish's last kernel is
                                          recorded under stage 3, a single launch only here) */
#define ADACOMP_STAGE_DECODE_CALL 8    /* a whole adacomp_decode_accumulate call */
#define ADACOMP_STAGE_DECODE_SGD_CALL 9  /* a whole adacomp_decode_sgd call (its kernels: stages 4-6) */
#define ADACOMP_STAGE_DECODE_ADAM_CALL 10 /* a whole adacomp_decode_adam call (its kernels: stages 4-6) */
#define ADACOMP_NUM_STAGES 11

/* A timer keeps the HIP events of every call recorded since the last read
 * (one per stage boundary); one timer may serve calls on several streams,
 * from one host thread at a time (it has no lock). */
int adacomp_timer_create(adacomp_timer** timer);
int adacomp_timer_destroy(adacomp_timer* timer);
/* Wait for every recorded event, then report per stage the summed
 * milliseconds and the number of launches since the last reset.  On
 * ADACOMP_ERR_HIP the calls read so far stay counted and the call whose
 * events failed is dropped. */
int adacomp_timer_read(adacomp_timer* timer, double* ms, uint64_t* launches, uint32_t nstages);
int adacomp_timer_reset(adacomp_timer* timer);

const char* adacomp_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ADACOMP_H */
