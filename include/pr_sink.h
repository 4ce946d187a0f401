/*
 * pr_sink.h -- C ABI of the PR-Sink bounded KV cache for AMD MI355X (gfx950).
 *
 * PR-Sink (Pose-Retrieval Sink attention, from LiveAnimate) lets the queries
 * of the current latent block attend over a cache of fixed size:
 *   Ref Sink     K/V of the reference image (always attended),
 *   Static Sink  K/V of the first generated block (kept for good),
 *   Dynamic Sink K/V of one earlier block recalled by pose retrieval,
 *   window       the W-1 blocks before the current one (W = 3 slots in all,
 *                the current block being the last slot),
 *   current      K/V of the block being denoised (passed by the caller).
 * Sources: HF papers abstract of LiveAnimate (Static/Dynamic Sink, three-slot
 * rolling window, memory and latency independent of stream length);
 * LiveAnimate review on paper.rainbus.top, full-pipeline paragraph (attention
 * formula over [K_ref; history; current], retrieval, Clean KV Update, RoPE
 * follow).
 *
 * Keys are stored raw (before RoPE) and attended rotated with 3D RoPE at their
 * *current* cache position ("RoPE follow"; review, full-pipeline and novelty
 * paragraphs).  Temporal positions are fixed by place: Ref at t0, then Static,
 * Dynamic, the previous window blocks (oldest first) and the current block,
 * each block_frames frames long; spatial positions are the latent (row,
 * column).  An empty segment is skipped and the others keep their positions.
 * The library rotates a block's raw keys once for every place the block takes
 * (Ref at set-up; block 0 at the Static place and a window block at each of
 * the W-1 window places it will take, all when its clean K/V are written; a
 * bank entry at the Dynamic place when written; the current block on every
 * attention call) and keeps the rotated copies next to the raw keys, so a key
 * is rotated once per place rather than once per query tile, and nothing is
 * rotated when the window slides.
 *
 * Memory: the caller allocates ONE device arena of pr_sink_arena_bytes(cfg)
 * bytes and every input/output tensor.  The library never allocates or frees
 * device memory; its footprint is fixed by the config and does not grow with
 * the stream.  Layout inside the arena is private, except as exposed by
 * pr_sink_slot_view().
 *
 * Tensor layout at the boundary: q, k, v, out are contiguous [T][H][d] in the
 * config's element type (bf16 or f32), T = block_frames*lat_h*lat_w tokens in
 * (frame, row, column) order; Ref tensors have T = ref_frames*lat_h*lat_w.
 * Every tensor pointer must be 16-byte aligned (PR_SINK_EINVAL otherwise).
 *
 * Streams: every call is asynchronous on `stream` (a hipStream_t passed as
 * void*; NULL = the null stream) except pr_sink_cache_init and
 * pr_sink_bank_state, which synchronise.  Inputs must stay valid until the
 * work queued on `stream` has run.  Calls may use different streams: the
 * library orders them with events (a stream waits only on work queued on
 * another stream that it depends on), so results do not depend on the
 * streams chosen.  The intended split (review, discussion of the Clean KV
 * Update's 24 % share: overlap it) puts pr_sink_clean_kv_write and
 * pr_sink_bank_update on a second stream.  A clean write of block b waits
 * only for block b's retrieval, the last bank update's copies and block b-1's
 * write of the same layer (it fills the slot of block b-W, which block b's
 * attention does not read), so it may overlap block b's attention; block
 * b+1's attention of layer l waits for block b's clean write of layer l; the
 * retrieval of block b+1 waits for block b's bank decision but not for the
 * copy of the entry it writes (that entry holds block b, which the retrieval
 * excludes), so the copy overlaps block b+1's attention.  The calls
 * themselves must come from one host thread, in the block order below.
 * The completion of pr_sink_attend is recorded on its stream only when a
 * call on another stream first has to wait for it, so a stream passed to
 * pr_sink_attend must stay alive until the next block's pr_sink_retrieve
 * returns.
 *
 * Call order per block b = 0, 1, 2, ...:
 *   pr_sink_retrieve(b)  ->  pr_sink_attend(layer) any number of times
 *   -> pr_sink_clean_kv_write(layer) once for every layer
 *   -> pr_sink_bank_update(b).
 * pr_sink_set_ref(layer) must have been called for every layer before block 0.
 * A call out of order returns PR_SINK_ESTATE.
 *
 * Errors: every int-returning call returns a pr_sink_status.  Arguments and
 * call order are validated before anything is queued, so an error leaves the
 * cache unchanged.  A HIP failure at launch returns PR_SINK_EHIP; the message
 * of the last failure on the calling thread is pr_sink_last_error().
 */
#ifndef PR_SINK_H_
#define PR_SINK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PR_SINK_OK = 0,
  PR_SINK_EINVAL = -1,   /* bad argument or config                          */
  PR_SINK_ESTATE = -2,   /* call out of order (block protocol)               */
  PR_SINK_ENOSPACE = -3, /* arena smaller than pr_sink_arena_bytes(cfg)      */
  PR_SINK_EHIP = -4      /* HIP runtime error, or the device is not gfx950   */
} pr_sink_status;

typedef enum { PR_SINK_BF16 = 0, PR_SINK_F32 = 1 } pr_sink_dtype;

/* Shape of one cache.  All fields are validated by every call that takes it. */
typedef struct pr_sink_config {
  int32_t n_layers;         /* >= 1; each layer has its own K/V in every slot       */
  int32_t n_heads;          /* >= 1                                                  */
  int32_t head_dim;         /* 64 or 128                                             */
  int32_t rope_dims[3];     /* (t, h, w) band widths: even, >= 2, sum == head_dim    */
  double rope_theta;        /* > 0; pair i of a D-wide band turns by pos*theta^(-2i/D) */
  int32_t lat_h, lat_w;     /* latent rows and columns per frame, >= 1              */
  int32_t ref_frames;       /* frames in the Ref Sink, >= 1                         */
  int32_t block_frames;     /* latent frames per block, >= 1                        */
  int32_t window_slots;     /* rolling-window slots including the current block, 1..5 */
  int32_t bank_size;        /* memory-bank entries M, 2..8                           */
  int32_t bank_fill_blocks; /* blocks b < this update the bank; later it is frozen   */
  int32_t fp_dim;           /* pose fingerprint length, 1..4096                      */
  int32_t dtype;            /* pr_sink_dtype of K/V/Q/out                            */
  int32_t t0;               /* temporal position of the first Ref frame, >= 0        */
  /* Bank-policy variants (review, weaknesses paragraph: directions for the
   * frozen bank and for failed pose detection), bits of pr_sink_bank_policy;
   * 0 = the method as described. */
  int32_t bank_policy;
  int32_t bank_stale_blocks; /* CONTINUAL: blocks an entry must go unused before it
                                may be evicted (its weight halves every this many
                                blocks, eviction at weight 1/2), >= 1              */
  double bank_refresh_tau;   /* GATED: refresh when the best dot product of the block's
                                fingerprint with the bank is below this, in [-1, 1] */
} pr_sink_config;

/* Bank-policy bits (pr_sink_config.bank_policy).
 *   ZERO_FALLBACK  a block whose fingerprint is all zero (every frame failed
 *                  detection) attends no Dynamic Sink (Static Sink + window
 *                  only) and is never written into the bank.
 *   CONTINUAL      past the fill phase the exhaustive replacement keeps
 *                  running, restricted to entries not written or retrieved in
 *                  the last bank_stale_blocks blocks (continual writes with
 *                  decaying weights).
 *   GATED          past the fill phase, a block whose best dot product with
 *                  the bank is below bank_refresh_tau triggers the full
 *                  exhaustive replacement (refresh gated by fingerprint
 *                  distance).
 * While the bank has room, any update inserts into the next slot. */
typedef enum {
  PR_SINK_BANK_ZERO_FALLBACK = 1,
  PR_SINK_BANK_CONTINUAL = 2,
  PR_SINK_BANK_GATED = 4
} pr_sink_bank_policy;

typedef struct pr_sink_cache pr_sink_cache; /* opaque, host-side handle */

/* Slot ids for pr_sink_slot_view.  PR_SINK_SLOT_DYNAMIC names the Dynamic
 * Sink, which has no storage of its own (it reads the bank entry that
 * pr_sink_retrieve returned); pr_sink_slot_view rejects it with
 * PR_SINK_EINVAL. */
enum {
  PR_SINK_SLOT_REF = 0,
  PR_SINK_SLOT_STATIC = 1,
  PR_SINK_SLOT_DYNAMIC = 2,
  PR_SINK_SLOT_WINDOW0 = 3 /* window slot j is PR_SINK_SLOT_WINDOW0 + j; bank entry i
                              follows the window: PR_SINK_SLOT_WINDOW0 + window_slots + i */
};

/* Bytes of device arena the config needs (0 if the config is invalid).
 * The method's cache is bounded: its memory does not grow with the length of
 * the stream (abstract on the HF papers page; jiazhuangai.com article, its
 * three key breakthroughs: a fixed memory overhead).  So this is a closed
 * form in the config only, and the arena is all the device memory the cache
 * ever uses. */
size_t pr_sink_arena_bytes(const pr_sink_config* cfg);

/* Creates the bounded cache of the method (HF papers abstract: sinks plus a
 * rolling window, in fixed memory; review on paper.rainbus.top, full-pipeline
 * paragraph: the Ref, Static and Dynamic Sinks and the window slots) over
 * `arena_dev` (device memory, >= pr_sink_arena_bytes(cfg) bytes, 256-byte
 * aligned; owned by the caller, must outlive the cache).
 * Clears the arena and uploads the RoPE cos/sin tables, then synchronises
 * `stream`.  With arena_dev == NULL and arena_bytes == 0 it creates a
 * dry-run cache that validates arguments and call order but never touches a
 * device.  *out receives the handle. */
int pr_sink_cache_init(const pr_sink_config* cfg, void* arena_dev, size_t arena_bytes,
                       void* stream, pr_sink_cache** out);

/* Writes the raw Ref Sink K and V of `layer` (device, [ref_T][H][d]) into the
 * cache (review, full-pipeline paragraph: K_ref, V_ref).  Allowed while no
 * block is open. */
int pr_sink_set_ref(pr_sink_cache* c, int32_t layer, const void* k_raw, const void* v_raw,
                    void* stream);

/* Opens block `block` (must be the next block).  Normalises the raw pose
 * fingerprint fp_raw_dev (device float[fp_dim]) to unit l2 norm in fp64 (an
 * all-zero fingerprint stays zero), scores it by dot product against every
 * bank entry whose block id is not block-1, takes the argmax (lowest slot on
 * ties), and makes that entry the block's Dynamic Sink (review, full-pipeline
 * paragraph: r(b) = argmax phi_b . phi_i excluding b-1, whose K/V go to the
 * Dynamic Sink; novelty paragraph: cosine similarity of l2-normalised
 * fingerprints).  Nothing is copied: attention reads bank entry r in place,
 * whose keys are kept rotated at the Dynamic Sink's place, and r stays on the
 * device (the host never waits for the retrieval).  The entry cannot change
 * while the block is open: the bank is written only by pr_sink_bank_update.
 * If no entry is eligible the Dynamic Sink is not attended during this block.
 * No key is rotated here: every window block's keys were rotated at all its
 * window places by its clean write.
 * slot_out_dev (device int32, nullable) receives the bank slot or -1. */
int pr_sink_retrieve(pr_sink_cache* c, int32_t block, const float* fp_raw_dev,
                     int32_t* slot_out_dev, void* stream);

/* One attention call of the open block for `layer`: rotates q and k_cur_raw
 * (device, [T][H][d], raw) at the current block's positions, takes every
 * cached key rotated at its segment's current position, and writes
 *   out = softmax(q_rot K_rot^T / sqrt(d)) V
 * over [Ref; Static; Dynamic; window; current] (review, full-pipeline
 * paragraph, attention formula; the current block attends to itself without
 * a mask).  k_cur_raw / v_cur_raw are the current block's raw K/V (device,
 * [T][H][d]); they are read, not stored.  out may not alias the inputs. */
int pr_sink_attend(pr_sink_cache* c, int32_t layer, const void* q_raw, const void* k_cur_raw,
                   const void* v_cur_raw, void* out, void* stream);

/* pr_sink_attend for callers that cannot allocate device memory or hand the
 * library a workspace (code under stream capture, tight serving loops): the
 * same call, except that the current block's rotated keys go to a static
 * device array of this library (64 MiB per GPU the library runs on, held
 * until the process ends) instead of the arena, and every attention job runs
 * whole (no split partial results).  Allocates nothing.  Returns
 * PR_SINK_EINVAL, leaving the cache unchanged, when the current block's keys
 * (block tokens x n_heads x head_dim x element size) exceed 64 MiB.  All calls
 * of this entry point on one GPU share the array: calls that may overlap on
 * one GPU (other streams, other caches, other threads) race and must not be
 * issued; each call overwrites what the previous one left there. */
int pr_sink_attend_noalloc(pr_sink_cache* c, int32_t layer, const void* q_raw, const void* k_cur_raw,
                           const void* v_cur_raw, void* out, void* stream);

/* Clean KV Update, write half: stores the clean raw K/V of the open block for
 * `layer` (device, [T][H][d]) into its rolling-window slot, and for block 0
 * also into the Static Sink (review, full-pipeline paragraph; HF abstract:
 * Static Sink = first generated block).  In the same pass it stores the keys
 * rotated at each of the W-1 window places the block takes from the next
 * block on (block 0 also at the Static Sink's place), so that opening a
 * block rotates nothing.  Once per layer per block. */
int pr_sink_clean_kv_write(pr_sink_cache* c, int32_t layer, const void* k_raw,
                           const void* v_raw, void* stream);

/* Closes block `block` (the open one; every layer must have been written).
 * While block < bank_fill_blocks, updates the memory bank: an empty entry is
 * filled with (block, phi_b, clean K/V); a full bank takes the option among
 * [keep, replace entry 0, ..., replace entry M-1] with the smallest mean
 * pairwise fingerprint similarity, keep winning ties (review, novelty
 * paragraph: exhaustive replacement minimising mean in-bank similarity;
 * weaknesses and reproducibility paragraphs: M = 5, frozen after 20 blocks). */
int pr_sink_bank_update(pr_sink_cache* c, int32_t block, void* stream);

/* Synchronises `stream` and copies the bank to host memory: ids_host
 * (int32[bank_size], -1 = empty), fp_host (double[bank_size*fp_dim], nullable),
 * misc_host (int32[3], nullable): {last retrieved slot or -1, block id held in
 * the Dynamic Sink or -1, last bank decision: -2 none, -1 keep, j >= 0 entry
 * written}. */
int pr_sink_bank_state(pr_sink_cache* c, int32_t* ids_host, double* fp_host,
                       int32_t* misc_host, void* stream);

/* Device pointers to the raw K, the V and the rotated K of one slot and
 * layer, for inspection.  All are [t_pad][H][d], token-major like the tensors
 * passed in; t_pad (a multiple of 64; the padding rows are zero) goes to
 * *t_pad_out.  Raw keys are kept only where a later rotation reads them: for
 * the Ref Sink, and for a window slot whose block may still enter the bank
 * (the fill phase, or the CONTINUAL and GATED policies), whose keys are then
 * rotated at the Dynamic Sink's place.  The Static Sink and bank entries are
 * attended rotated only.  *k_dev receives NULL where no raw keys are kept.
 * The rotated K holds the keys rotated at the place the slot's block takes in
 * the window of the open block (of the next one between blocks); for the
 * block written in it, or one that has left the window, the newest window
 * place.  Static: at the Static Sink's place; a bank entry: at the Dynamic
 * Sink's place.  k_rot_dev may be NULL.  PR_SINK_SLOT_DYNAMIC is rejected
 * (PR_SINK_EINVAL): view the bank entry the open block retrieved instead. */
int pr_sink_slot_view(const pr_sink_cache* c, int32_t slot, int32_t layer, void** k_dev,
                      void** v_dev, void** k_rot_dev, int32_t* t_pad_out);

/* Measurement hook: with events set (hipEvent_t passed as void*, created by
 * the caller with timing enabled), every later pr_sink_attend records
 * ev_start on its stream right before its attention kernel and ev_stop right
 * after it, so the kernel's own duration can be read without the rotation of
 * the current keys that precedes it.  Both NULL turns it off.  The events
 * stay owned by the caller and must outlive their use. */
int pr_sink_set_attend_events(pr_sink_cache* c, void* ev_start, void* ev_stop);

/* Segments of the open block in cache order (Ref, Static, Dynamic, W-1
 * window blocks oldest first, current): token counts (0 = not attended) and
 * temporal start of each, n_out receives the count (window_slots + 3). */
int pr_sink_segments(const pr_sink_cache* c, int32_t* tokens_out, int32_t* t_start_out,
                     int32_t* n_out);

/* Frees the host-side handle (never the arena). */
int pr_sink_cache_destroy(pr_sink_cache* c);

/* Message of the last error on the calling thread ("" if none). */
const char* pr_sink_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PR_SINK_H_ */
