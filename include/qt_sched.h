/* qt_sched.h -- host lockstep scheduler around the decode frame (qt.h), in libqt.so.
 *
 * Sessions are decoded one frame at a time in lockstep: qt_sched_step decodes one
 * frame for every session with a queued input, in as few batched frame calls as
 * the captured batch sizes allow.  Sources:
 *  - "Qwen3-TTS Native v0.3.0", What changed: one batched call runs the frame for
 *    every active session; the frame is captured once per session tuple and
 *    replayed; a session's first frame does not wait for the lockstep rendezvous.
 *  - decomputer.nl article on Qwen3-TTS serving, section 5: graphs are captured for
 *    a fixed set of batch sizes and a ready group larger than the largest one is
 *    split over several scheduling turns; the termination check is deferred while
 *    end of speech is suppressed, so the host can queue further work without
 *    waiting for the device.
 *
 * Behaviour
 *  - Grouping: ready sessions fall into classes (first frame or not, teacher-forced
 *    or not, sampling or not); classes never share a batched call, first-frame
 *    classes run first.
 *    Each class is cut into groups of the largest captured size plus one remainder
 *    group, and each group replays the graph of the smallest captured size that
 *    holds it; the extra slots (padding) decode a zero input into a reserved page
 *    and nothing of theirs reaches a session.
 *  - Pages: the Talker KV pool `kv` belongs to the scheduler.  Its last page is
 *    reserved for padding slots; the others form the free list.  qt_sched_open
 *    hands a new session the pages for its prefilled positions (the caller then
 *    writes its prefill into them), and qt_sched_step appends one page whenever a
 *    session's next position starts a new page.  A closed session's pages and id
 *    return to the free lists once the device has finished its last frame, which
 *    the scheduler learns from an event per step (it never waits for one, except
 *    that a step waits for the step 64 before it when the host runs that far ahead).
 *  - End of speech (eos_index >= 0): from its min_frames-th frame on, the frame
 *    ends the session when the end-of-speech entry of logits0 would win the
 *    codebook-0 choice, i.e. the argmax over [0, cb0_range) plus that entry, lowest
 *    index winning ties.  The device decides this and writes the ending frame's
 *    number into the caller's pinned host buffer; earlier frames write nothing, and
 *    the host reads the buffer without waiting (qt_sched_state).  A session also
 *    ends when it has decoded max_frames frames.
 *  - Per-session outputs of the last decoded frame are copied to per-session slots
 *    of the device buffer, so every call's results stay readable after the shared
 *    batch buffers are reused by the next group.
 *  - Device memory is the caller's (qt_sched_bytes); the library allocates none.
 *    Every step enqueues only on the scheduler's stream.  Frames of different
 *    schedulers, or a qt_frame_decode sharing the KV pool, must be ordered by the
 *    caller.
 *
 * Errors are qt_status codes (qt.h) with qt_last_error() text; a call that fails
 * its host checks changes nothing and enqueues nothing. */
#ifndef QT_SCHED_H
#define QT_SCHED_H

#include "qt.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qt_sched qt_sched;

#define QT_SCHED_MAX_BUCKETS 8
#define QT_SCHED_MAX_BATCH 32
#define QT_SCHED_MAX_SESSIONS 4096

typedef struct {
  int32_t n_buckets;                     /* 1..QT_SCHED_MAX_BUCKETS */
  int32_t buckets[QT_SCHED_MAX_BUCKETS]; /* captured batch sizes, strictly ascending,
                                            1..QT_SCHED_MAX_BATCH */
  int32_t max_sessions;                  /* sessions open at once, 1..QT_SCHED_MAX_SESSIONS */
  int32_t max_pages;                     /* page-table row length per session, >= 1 */
  int32_t eos_index;                     /* logits0 entry of end of speech in [0, talker_vocab),
                                            or -1: sessions end only at max_frames */
} qt_sched_cfg;

typedef enum {
  QT_SESSION_FREE = 0,      /* not open */
  QT_SESSION_RUNNING = 1,   /* open and not known to have ended */
  QT_SESSION_ENDED_EOS = 2, /* a decoded frame chose end of speech */
  QT_SESSION_ENDED_MAX = 3  /* it has been given max_frames frames */
} qt_session_state;

/* Bytes of the device buffer (256-byte aligned) and of the pinned host buffer that
 * qt_sched_create needs for this model configuration and scheduler configuration.
 * Host-only; QT_E_SHAPE / QT_E_INVALID_ARG for configurations it rejects. */
qt_status qt_sched_bytes(const qt_model_cfg* model_cfg, const qt_sched_cfg* cfg,
                         uint64_t* device_bytes, uint64_t* host_bytes);

/* Create a scheduler over `model` and the Talker KV pool `kv` (num_pages >= 2; all
 * pages start free).  `device_buf`: device memory of qt_sched_bytes' device size;
 * `host_buf`: pinned, device-mapped host memory (hipHostMalloc) of its host size,
 * 16-byte aligned.  Both stay the caller's and must outlive the scheduler.
 * `stream`: the hipStream_t every step enqueues on (its status word is cleared
 * there now).  Graphs are captured on a step's first use of a batch size. */
qt_status qt_sched_create(qt_model* model, const qt_sched_cfg* cfg, const qt_kv_caches* kv,
                          void* device_buf, uint64_t device_bytes, void* host_buf,
                          uint64_t host_bytes, void* stream, qt_sched** out);

/* Open a session whose Talker cache will hold `length` prefilled positions
 * (0 <= length < max_pages * page_size).  It receives ceil(length / page_size)
 * pages from the free list, written in position order to `pages` (host int32 array
 * of at least that many entries; may be NULL when length is 0); the caller stores
 * the prefilled keys and values there before the session's first step.  It ends at
 * end of speech from its min_frames-th frame on (min_frames >= 1), or after
 * max_frames >= 1 frames.  *session receives its id in [0, max_sessions).
 * QT_E_CAPACITY if max_sessions are open (closed ones count until the device is
 * done with them) or too few pages are free. */
qt_status qt_sched_open(qt_sched* s, int32_t length, int32_t min_frames, int32_t max_frames,
                        int32_t* pages, int32_t* session);

/* Draw the session's tokens (qt_sampling in qt.h) from its next submitted frame on:
 * params (host [2]: codebook 0, then the predictor's codebooks) and seed are copied
 * now; params = NULL returns the session to greedy tokens.  The draw counter is the
 * session's cache length before each frame, and its seen set of codebook-0 tokens
 * starts empty at open.  Sampling and greedy sessions are decoded in separate
 * batched calls.  End of speech is still decided against the greedy codebook-0
 * choice.  QT_E_INVALID_ARG for parameters out of range. */
qt_status qt_sched_set_sampling(qt_sched* s, int32_t session, const qt_sampler_params* params,
                                uint64_t seed);

/* Queue the next frame of a running session.  talker_in: device bf16 [talker hidden];
 * forced: device int32 [n_codebooks] or NULL (teacher forcing as in qt_frame_inputs).
 * Both are read by the device when the frame runs, so they stay valid until then.
 * QT_E_STATE if the session is not running (ended, as far as the host knows, or not
 * open) or already has a frame queued. */
qt_status qt_sched_submit(qt_sched* s, int32_t session, const void* talker_in,
                          const int32_t* forced);

/* Decode every queued frame (enqueue only).  *n_groups (may be NULL) receives the
 * number of batched frame calls made.  QT_E_CAPACITY, with nothing enqueued, if a
 * session would grow past max_pages or the free list is short of new pages;
 * QT_E_HIP if a graph capture fails. */
qt_status qt_sched_step(qt_sched* s, int32_t* n_groups);

/* Device pointers to the session's outputs of its last decoded frame: logits0 f32
 * [talker_vocab], logits_pred f32 [n_codebooks-1][code_vocab], tokens int32
 * [n_codebooks].  They are overwritten by its next frame (stream-ordered).  *frames
 * receives the number of frames decoded (any output pointer may be NULL). */
qt_status qt_sched_outputs(qt_sched* s, int32_t session, const float** logits0,
                           const float** logits_pred, const int32_t** tokens, int32_t* frames);

/* The session's qt_session_state as far as the host knows without waiting, and
 * *end_frame (may be NULL): the 1-based number of the frame that ended it, else 0.
 * Frames queued after the ending one, before the host knew, are to be discarded. */
qt_status qt_sched_state(qt_sched* s, int32_t session, int32_t* state, int32_t* end_frame);

/* Positions in the session's Talker cache once its decoded frames have run. */
qt_status qt_sched_length(qt_sched* s, int32_t session, int32_t* length);

/* Device uint32 word into which every frame ORs its QT_STATUS_* bits (qt.h). */
qt_status qt_sched_status_word(qt_sched* s, uint32_t** status);

/* Pages currently on the free list (closed sessions' pages count once released). */
qt_status qt_sched_free_pages(qt_sched* s, int32_t* n);

/* Close a session (a queued frame is dropped).  Its id and pages are reused once the
 * device has finished its last frame; the call never waits for that. */
qt_status qt_sched_close(qt_sched* s, int32_t session);

/* The grouping qt_sched_step uses, as a pure host function: n ready sessions with
 * classes cls[i] >= 0 (sessions of different classes never share a group; lower
 * classes run first; within a class, input order).  group_of[i] (host, n entries)
 * receives session i's group, group_bucket[g] (host, room for n entries) the
 * captured size group g replays, *n_groups the number of groups.  buckets: as in
 * qt_sched_cfg. */
qt_status qt_sched_plan(const int32_t* cls, int32_t n, const int32_t* buckets,
                        int32_t n_buckets, int32_t* group_of, int32_t* group_bucket,
                        int32_t* n_groups);

/* Wait for the scheduler's last step to finish, then release its graphs and events. */
void qt_sched_destroy(qt_sched* s);

#ifdef __cplusplus
}
#endif
#endif
