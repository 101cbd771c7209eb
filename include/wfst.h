/*
 * wfst.h -- C ABI of the MI355X (gfx950) WFST Viterbi beam-search decoder.
 *
 * The decoder takes per-frame CTC log-posteriors log_prob[B, T, V] and a CSR
 * decoding graph (epsilon-free HLG-style, or TLG-style with epsilon arcs) and
 * returns, per utterance, the best word sequence, the arc ids of the best path
 * and its score. Semantics follow the page "GPU WFST Beam-Search Decoder" (OASR
 * docs): section 1 "Purpose and Responsibilities" (relaxation
 * end = score[src] + arc_weight + log_prob[t][ilabel], recombination by
 * destination, backtrack through arc ids to words), section 3 "Decoding
 * Semantics" (dynamic beam, soft max_active, exact admit test, final step,
 * allow_partial), section 5.3 (fp32 addition order (score + weight) + log_prob),
 * section 5.5 (epsilon closure), section 7 (outputs, overflow bits) and
 * section 10 "Public C API" (load graph / create decoder / decode batch / free,
 * out_meta = {ok, reached_final, overflow}). Among equal scores the smallest arc
 * id wins, so results are deterministic.
 *
 * Conventions for every call: the return value is 0 (WFST_OK) or a negative
 * status; on failure wfst_last_error() returns a message for the calling
 * thread. Host pointers are only read during the call unless stated.
 */
#ifndef WFST_H
#define WFST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WFST_OK        0
#define WFST_EINVAL   -1   /* an argument is out of range or a pointer is null       */
#define WFST_ECORRUPT -2   /* the graph fails validation (nothing was uploaded)      */
#define WFST_ENOMEM   -3   /* a device or host allocation failed                     */
#define WFST_EDEVICE  -4   /* a HIP runtime call failed (no device, launch failure)  */

#define WFST_LP_F32 0      /* log_prob elements are binary32                          */
#define WFST_LP_F16 1      /* log_prob elements are binary16, widened exactly to fp32 */

/* out_meta[b * 3 + 2] bits (section 7 of the page): a non-zero value means the
 * lane's result may be degraded; such a lane also reports ok = 0. */
#define WFST_OVF_SLOTS    1   /* a lane's candidate arcs in one step exceed slot_cap       */
#define WFST_OVF_HASH     2   /* recomb_slots > 0: more distinct destinations in one pass than the hash holds */
#define WFST_OVF_ARENA    4   /* the lane's winners-log region is full                     */
#define WFST_OVF_CLAIMS   8   /* more admitted candidates in one pass than claims_cap      */
#define WFST_OVF_FRONTIER 16  /* more surviving tokens than frontier_cap                   */
#define WFST_OVF_PATH     32  /* best path longer than the device path buffer              */

typedef struct wfst_graph_s *wfst_graph_t;
typedef struct wfst_decoder_s *wfst_decoder_t;

/*
 * A decoding graph in CSR form, as host arrays (page section 4 "Graph Image":
 * row_splits, per-arc destination, ilabel, word label and weight; arc order is
 * identity: arc id = CSR index, never reordered).
 *
 *  num_states   states including the super-final state, which must be the last
 *               state (num_states - 1) and have no out-arcs; >= 2.
 *  num_arcs     total arcs, including final arcs; in [0, 2^31 - 1).
 *  start_state  in [0, num_states - 1).
 *  vocab_size   V: width of a log_prob row; in [1, 65535) (ilabels are stored as
 *               u16 on the device, page section 4).
 *  epsilon_id   -1 when the graph has no epsilon arcs; otherwise the ilabel that
 *               marks an epsilon arc, in [0, V) (0 on TLG graphs); that column
 *               of log_prob is then never read.
 *  row_splits   [num_states + 1], row_splits[0] = 0, non-decreasing,
 *               row_splits[num_states] = num_arcs.
 *  dest         [num_arcs], in [0, num_states).
 *  ilabel       [num_arcs]: -1 for a final arc, epsilon_id for an epsilon arc,
 *               else an emitting label in [0, V).
 *  olabel       [num_arcs]: word id, 0 = no word; >= 0.
 *  weight       [num_arcs]: log-score added to the path score; NaN and +inf are
 *               rejected.
 * Per state the arcs must come as [epsilon arcs][emitting arcs][final arcs];
 * an arc enters the super-final state iff it is a final arc.
 */
typedef struct wfst_graph_desc {
    int32_t num_states;
    int32_t num_arcs;
    int32_t start_state;
    int32_t vocab_size;
    int32_t epsilon_id;
    const int32_t *row_splits;
    const int32_t *dest;
    const int32_t *ilabel;
    const int32_t *olabel;
    const float *weight;
} wfst_graph_desc;

/*
 * Search settings (page section 10, wfst_create_decoder; section 3 for the
 * meaning of beam, min_active, max_active and allow_partial).
 *
 *  beam            search beam (> 0, finite).
 *  min_active      lower frontier target of the dynamic beam (>= 0; 0 default).
 *  max_active      upper frontier target, enforced only through beam decay (>= 1).
 *  allow_partial   1: when no frontier state has a final arc on the last step,
 *                  the best-scoring token ends the path (reached_final = 0).
 *  max_lanes       largest batch B a decode may use; in [1, 64].
 *  max_frames      largest T a decode may use; >= 1.
 *  lp_dtype        WFST_LP_F32 or WFST_LP_F16.
 *  eps_iterations  epsilon-closure passes after each real step (and once on the
 *                  start frontier); ignored on graphs without epsilon arcs;
 *                  in [0, 16].
 *  use_graphs      1: each decode replays one captured hipGraph of the whole
 *                  frame loop; 0: plain launches (same kernels, same results).
 *  frontier_cap    tokens per lane per step (0: 64 * max_active);
 *                  frontier_cap * (largest out-degree of one arc class) must
 *                  stay below 2^32.
 *  claims_cap      admitted candidates per lane per pass
 *                  (0: min(slot_cap, max(frontier_cap, 2^20))); in [1, 2^28].
 *  arena_entries   winners-log entries per lane per decode
 *                  (0: 4 * max_active * (max_frames + 2) * (1 + eps passes),
 *                  at least 2^20); max_lanes * arena_entries < 2^31.
 *  grid_blocks     workgroups per launch of the frame-loop kernels (0: derive: up to
 *                  4 per CU, the slot walk up to 5 per CU, fewer for small batches).
 *  slot_cap        candidate arcs (slots) per lane per step (0: 512 * max_active,
 *                  at least 2^16); at most 2^31.
 *  plain_keys      0: the recombination table's keys carry the round's epoch
 *                  in the bits their tie part leaves free, so entries are never
 *                  cleared one by one. The tie part is the arc's rank among its
 *                  destination's incoming arcs (ordered as the arc ids are)
 *                  when the graph upload could store the ranks (state id bits +
 *                  rank bits <= 31), else the arc's record position on the
 *                  device (graphs of at most 2^25 arc records: the arcs and up
 *                  to 31 padding records per state, which order arcs as their
 *                  ids do). Rounds are numbered on across decodes and stream
 *                  calls, and the table is wiped before the first round past
 *                  each multiple of the epoch period (epoch_period).
 *                  2: the same with arc id ties. 1: plain keys, each entry
 *                  cleared by its owner (also what 0 and 2 fall back to when
 *                  the tie part needs more than 25 bits). Same results.
 *  path_cap        arcs of a result path kept per lane (0: (max_frames + 2) *
 *                  (1 + eps passes)); in [0, 2^26]. A longer path keeps its
 *                  newest path_cap arcs (its words are those arcs' words) and
 *                  sets WFST_OVF_PATH. A stream's path spans all its frames
 *                  (section 8): size this for the longest stream.
 *  lattice         1: lattice mode (section 1 "Lattice mode", section 7
 *                  "Lattice"): every admitted candidate of every step is kept
 *                  as a lattice arc, and on graphs with epsilon arcs every
 *                  epsilon candidate a closure pass admits (section 5.5: the
 *                  candidate set persisted after the closure, epsilon arcs
 *                  tagged), as an arc inside the frame the closure prepares;
 *                  after the decode a backward pass prunes them with
 *                  output_beam (section 3); read the result with
 *                  wfst_lattice_records. On graphs with epsilon arcs every
 *                  epsilon weight must be <= 0. No streams.
 *  output_beam     the lattice prune's beam (finite, >= 0): an arc survives iff
 *                  (fwd(src) + s) + bwd(dst) >= best - output_beam, with s the
 *                  arc's own score (weight + log-prob; a final or epsilon arc's
 *                  weight; 0 for the redirect's virtual arc), fwd the score of
 *                  its source token after the frame's closure, bwd(token) the
 *                  best continuation to the super-final state (s + bwd(dst)
 *                  maximised over its arcs, last frame first; inside a frame,
 *                  over its epsilon arcs, to a fixpoint), best the lane's result
 *                  score; binary32, in that order.
 *  lattice_cap     lattice arcs held (and kept records) per lane per decode
 *                  (0: 2 * max_active * (max_frames + 2), at least 2^20); in
 *                  [0, 2^28]. More sets WFST_OVF_ARENA (the 1-best result is
 *                  still exact). A lattice also holds max(arena_entries,
 *                  lattice_cap) + 1 nodes (tokens) per lane; more (possible
 *                  only with gc_interval > 0) sets the same bit.
 *  lat_prune_interval  0: none. N in [1, 512] (lattice mode): section 7's
 *                  interval prune, window-loose: after every N steps that are
 *                  not a lane's last, backward scores over the last 2N frames
 *                  are computed from -fwd at the frontier (no complete path
 *                  through a frontier token can beat the final best), and arcs
 *                  with (fwd(src) + s) + bwd(dst) < 0 - output_beam are dropped
 *                  (the final test could not keep them, in exact arithmetic);
 *                  lattice_cap then bounds the arcs held at once, not all
 *                  admitted ones. The final pass is unchanged.
 *  gc_interval     0: the winners log keeps every entry of a decode (arena_entries
 *                  per lane must hold them all). n > 0: after every n steps, and
 *                  at the end of each stream chunk, a compaction round keeps only
 *                  the entries a live token still reaches (page section 8.1):
 *                  the log then holds the path all tokens share (about one entry
 *                  per frame) plus the recent tree, so a small arena_entries
 *                  serves long utterances and streams. Results are identical.
 *                  Lattice mode may use it (lattice nodes are frame positions,
 *                  never log entries). With n > 0 arena_entries defaults to
 *                  max(2^20, 8 * max_active * (n + 2) * (1 + eps passes)).
 *  arena_commit    how much of the winners-log regions is backed by memory
 *                  (page section 6.2, lazily committed regions): the whole
 *                  max_lanes * arena_entries range is reserved as address space
 *                  at creation, and 4 MiB chunks are mapped behind it as lanes
 *                  need them. 0: commit min(arena_entries, 2^19) entries per lane
 *                  first; n > 0: min(arena_entries, n) first; -1: one plain
 *                  allocation of the whole range (as on a device without virtual
 *                  memory management, where the others do the same). A decode in
 *                  which a lane outgrows the committed part commits more (at
 *                  least double, aimed at the longest lane's end) and runs again
 *                  on the same inputs, so results are those of a fully committed
 *                  region; wfst_decoder_stats reports the re-runs. Creating a
 *                  stream commits its own lane's whole region when it opens (it
 *                  cannot run again), so committed memory grows with the
 *                  streams opened; chunks stay mapped after release.
 *  recomb_slots    0: recombination through a direct-mapped table of one 8-byte
 *                  key per state and lane (max_lanes * num_states * 8 bytes,
 *                  twice on graphs with epsilon arcs and eps_iterations > 0: a
 *                  closure pass resolves from one while the next relaxes into
 *                  the other; no probing, never full). n > 0, a power of 2 in
 *                  [64, 2^28]: a per-lane open-addressing hash of n 16-byte
 *                  slots keyed on the destination state (page section 5.3's
 *                  hash; memory max_lanes * n * 16 bytes, twice likewise,
 *                  independent of the graph's size), claimed
 *                  with a CAS and resolved with the same 64-bit atomicMax; a pass
 *                  with more distinct destinations than n retires the lane with
 *                  WFST_OVF_HASH. Same results. Needs epoch keys (plain_keys != 1).
 *  epoch_period    recombination rounds between table wipes with epoch keys
 *                  (0: derive: 2^(32 - tie bits) - 1, at most 65535); n in
 *                  [2, that value]: wipe more often (same results).
 */
typedef struct wfst_decoder_config {
    float beam;
    int32_t min_active;
    int32_t max_active;
    int32_t allow_partial;
    int32_t max_lanes;
    int32_t max_frames;
    int32_t lp_dtype;
    int32_t eps_iterations;
    int32_t use_graphs;
    int32_t frontier_cap;
    int32_t claims_cap;
    int32_t grid_blocks;
    int64_t arena_entries;
    int64_t slot_cap;
    int32_t plain_keys;
    int32_t path_cap;
    int32_t lattice;
    float output_beam;
    int64_t lattice_cap;
    int32_t gc_interval;
    int64_t arena_commit;
    int32_t epoch_period;
    int32_t lat_prune_interval;
    int64_t recomb_slots;
} wfst_decoder_config;

/* Message of the last failed call on this thread ("" if none). The pointer stays
 * valid until the next call on the same thread. */
const char *wfst_last_error(void);

/*
 * Validate a host CSR graph and upload it to `device` (page section 4: the
 * loader validates every index the decoder later follows; the device copy is
 * split into per-arc columns, ilabel as u16, and per-state arc ranges and the
 * largest emitting / final weight of each state are computed once here).
 * The host arrays are copied; the caller may free them when the call returns.
 * On success *out holds one reference; release it with wfst_graph_release.
 * Errors: WFST_EINVAL (null pointer, bad device), WFST_ECORRUPT (any rule of
 * wfst_graph_desc broken; checked before any device work), WFST_ENOMEM,
 * WFST_EDEVICE.
 */
int wfst_graph_upload(const wfst_graph_desc *g, int device, wfst_graph_t *out);

/* Drop one reference (page section 10: a decoder co-owns its graph, so the
 * graph may be released before its decoders). Null is a no-op. */
int wfst_graph_release(wfst_graph_t g);

/*
 * Create a decoder on the graph's device: allocates every workspace buffer once
 * (frontiers, per-lane recombination tables, claims lists, winners-log regions,
 * result buffers) and takes a graph reference (page section 6.1 "Workspace",
 * section 10). The recombination table holds one 8-byte entry per state and
 * lane (max_lanes * num_states * 8 bytes; two tables when closure passes run),
 * so destinations are resolved with one atomic each and never overflow (or,
 * with recomb_slots, a per-lane hash).
 * Errors: WFST_EINVAL (bad config),
 * WFST_ENOMEM, WFST_EDEVICE.
 */
int wfst_decoder_create(wfst_graph_t g, const wfst_decoder_config *c, wfst_decoder_t *out);

/*
 * Decode a batch (page section 10 wfst_decode_batch, section 7 outputs).
 *
 *  log_prob      device pointer to a packed [B, T, V] tensor of lp_dtype on the
 *                decoder's device (row (b, t) at log_prob + (b*T + t)*V); owned
 *                by the caller and left untouched; must stay valid until the
 *                call returns.
 *  B, T, V       1 <= B <= max_lanes, 0 <= T <= max_frames, V = graph vocab_size.
 *  lengths_host  [B] host int32, each in [0, T]; frames t >= lengths[b] of lane b
 *                are never read.
 *  stream        the caller's HIP stream (hipStream_t; null = the null stream):
 *                the decode is ordered after work already queued on it, and the
 *                call returns after synchronising it once, when the results
 *                have been copied back.
 *  out_words     [B * words_cap] host: lane b's word ids at b*words_cap.
 *  out_word_lens [B] host: TRUE word counts (may exceed words_cap; the first
 *                words_cap words are written).
 *  out_arcs      [B * arcs_cap] host: arc ids of the best path in forward order,
 *                epsilon and final arcs included.
 *  out_arc_lens  [B] host: TRUE path lengths (may exceed arcs_cap).
 *  out_scores    [B] host: best path score (binary32); -inf when the lane has no
 *                path.
 *  out_meta      [B * 3] host: {ok, reached_final, overflow bits}.
 * out_words / out_arcs may be null when their cap is 0. A lane with no path
 * (every candidate of a real step pruned or no arc to expand, or no final arc on
 * the last step without allow_partial) reports ok = 1, reached_final = 0,
 * score -inf and no arcs. The call is idempotent and serial per decoder (an
 * internal mutex); other decoders may run concurrently.
 * Errors: WFST_EINVAL (ranges above, null pointers, V mismatch, the decoder
 * holds open streams, or log_prob is not device memory of the decoder's device
 * or ends before B * T * V elements), WFST_EDEVICE.
 */
int wfst_decode(wfst_decoder_t d, const void *log_prob, int32_t B, int32_t T, int32_t V,
                const int32_t *lengths_host, void *stream,
                int32_t *out_words, int32_t words_cap, int32_t *out_word_lens,
                int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens,
                float *out_scores, int32_t *out_meta);

/* Free the decoder's workspace and its graph reference. Null is a no-op. */
int wfst_decoder_destroy(wfst_decoder_t d);

/*
 * For callers that cannot allocate device memory (code that runs under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): one
 * decode, as wfst_decode, of the batch with the decoder configuration *c, that
 * calls no hipMalloc, hipFree or other allocating routine. There is no decoder
 * object: every workspace buffer of the decode (control blocks, frontiers,
 * candidate list, recombination table, winners log, results) is laid out in a
 * static device scratch of WFST_NOALLOC_SCRATCH_BYTES (64 MiB) per device,
 * which each device the library runs on holds until the process ends.
 *
 *  g             an uploaded graph (wfst_graph_upload), on the device the call
 *                runs on; the call takes no reference.
 *  c             the same fields as wfst_decoder_create's (0 = derive a
 *                capacity the same way); lattice and gc_interval must be 0,
 *                use_graphs and arena_commit are ignored (plain launches, the
 *                whole winners-log region backed). The workspace these sizes
 *                give must fit the scratch, else WFST_EINVAL with the bytes
 *                needed: the derived defaults suit decoder objects and are far
 *                larger, so callers set frontier_cap, claims_cap, slot_cap,
 *                arena_entries (and path_cap) for their batches.
 *  log_prob ...  as wfst_decode (B <= max_lanes, T <= max_frames). A lane whose
 *                winners log outgrows arena_entries reports WFST_OVF_ARENA (no
 *                region can grow here). In out_words / out_arcs, entries past a
 *                row's length (up to its cap) are unspecified.
 * Results equal wfst_decode's for the same graph, config and inputs. Calls on
 * one device share its scratch and its contents from the previous call: they
 * run one at a time (a process-wide lock per device; the call returns after
 * synchronising `stream`), and every call clears what must start empty. Calls
 * from separate processes use separate scratch copies.
 * Errors: WFST_EINVAL (as wfst_decode, lattice or gc_interval set, workspace
 * larger than the scratch), WFST_EDEVICE.
 */
#define WFST_NOALLOC_SCRATCH_BYTES (64ll << 20)
int wfst_decode_noalloc(wfst_graph_t g, const wfst_decoder_config *c, const void *log_prob, int32_t B, int32_t T,
                        int32_t V, const int32_t *lengths_host, void *stream,
                        int32_t *out_words, int32_t words_cap, int32_t *out_word_lens,
                        int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens,
                        float *out_scores, int32_t *out_meta);

/*
 * Streams (page section 8 "Streaming Lifecycle", section 3 on the online beam):
 * a stream decodes one utterance whose frames arrive in chunks. It holds one
 * lane of the decoder from wfst_create_stream to wfst_release_stream; its search
 * state stays on the device between calls. Until wfst_finalize_stream the
 * utterance length counts as unbounded, so the raise of min_active over an
 * utterance's last frames never applies (k2's online semantics); any chunking
 * of the same frames gives the same search. A stream's whole path stays in its
 * lane's winners-log region (arena_entries entries): a longer stream overflows
 * it (WFST_OVF_ARENA). max_frames bounds one chunk, not the stream. While any
 * stream is open, wfst_decode is refused. All calls are serial per decoder.
 */

/*
 * Open a stream: *channel = the lane it holds, or -1 when every lane holds one
 * (not an error). Runs the start frontier's epsilon closure for that lane only.
 * Errors: WFST_EINVAL (null, lattice mode), WFST_EDEVICE.
 */
int wfst_create_stream(wfst_decoder_t d, void *stream, int32_t *channel);

/*
 * Open up to n streams in one call (one device sequence for all of them):
 * channels[0 .. *opened) receive their lanes, the lowest free lanes first;
 * *opened < n when fewer lanes are free (not an error). channels holds n
 * entries. Errors: WFST_EINVAL (null, n < 0, lattice mode), WFST_EDEVICE.
 */
int wfst_create_streams(wfst_decoder_t d, int32_t n, void *stream, int32_t *channels, int32_t *opened);

/*
 * Advance C open streams by one chunk each.
 *  channels      [C] host: distinct open channels, 1 <= C <= max_lanes.
 *  log_prob      device pointer to a packed [C, T, V] tensor of lp_dtype: row j
 *                holds channels[j]'s next frames; owned by the caller and left
 *                untouched; must stay valid until the call returns.
 *  T, V          0 <= T <= max_frames, V = graph vocab_size.
 *  lengths_host  [C] host: frames of each channel's chunk, in [0, T].
 *  stream        the caller's HIP stream; the call returns after synchronising it.
 *  want_partial  non-zero: write each channel's partial hypothesis (the path of
 *                its best current token: greatest (score, then smallest arc id
 *                of the arc that gave the token its score)) to the outputs,
 *                laid out as wfst_decode's for B = C, row j for channels[j], with
 *                reached_final = 0 (score -inf and no arcs once the stream's
 *                search has died). Otherwise the outputs are not touched and may
 *                be null.
 * Errors: WFST_EINVAL (ranges above, a channel not open or repeated, null
 * pointers, log_prob not device memory of the decoder's device or shorter than
 * C * T * V elements), WFST_EDEVICE.
 */
int wfst_advance_chunk(wfst_decoder_t d, const int32_t *channels, int32_t C, const void *log_prob,
                       int32_t T, int32_t V, const int32_t *lengths_host, void *stream,
                       int32_t want_partial, int32_t *out_words, int32_t words_cap,
                       int32_t *out_word_lens, int32_t *out_arcs, int32_t arcs_cap,
                       int32_t *out_arc_lens, float *out_scores, int32_t *out_meta);

/*
 * End a stream: its utterance length becomes the frames it has received, the
 * final step runs (final arcs, beam 1e10, redirect with allow_partial) and the
 * result is written as wfst_decode's for one lane. The channel stays held (a
 * second call returns the same result) until released.
 * Errors: WFST_EINVAL (channel not open, null pointers), WFST_EDEVICE.
 */
int wfst_finalize_stream(wfst_decoder_t d, int32_t channel, void *stream, int32_t *out_words,
                         int32_t words_cap, int32_t *out_word_len, int32_t *out_arcs, int32_t arcs_cap,
                         int32_t *out_arc_len, float *out_score, int32_t *out_meta);

/*
 * End several streams in one call: one device sequence serves them all (the
 * final step of every listed lane at once, then their paths), which a serving
 * loop ending many utterances together pays once instead of per stream.
 * channels[j], j < C, are distinct open channels; row j of the outputs receives
 * channels[j]'s result exactly as wfst_finalize_stream writes it (words and
 * arcs rows of words_cap / arcs_cap entries).
 * Errors: WFST_EINVAL (C outside [1, max_lanes], a channel not open or
 * repeated, null pointers), WFST_EDEVICE.
 */
int wfst_finalize_streams(wfst_decoder_t d, const int32_t *channels, int32_t C, void *stream,
                          int32_t *out_words, int32_t words_cap, int32_t *out_word_lens,
                          int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens, float *out_scores,
                          int32_t *out_meta);

/* Give a stream's lane back (no device work). Errors: WFST_EINVAL (not open). */
int wfst_release_stream(wfst_decoder_t d, int32_t channel);

/*
 * Blank-skip frame pre-slicing before a decode (page section 3: a step before
 * the search, as WeNet slices frames, with 0.98 as the usual threshold): frame t < lengths[b] of
 * lane b is dropped iff its blank probability exceeds `threshold`, tested in
 * binary32 as log_prob[b, t, blank_id] > (float) log(threshold); the kept rows
 * keep their order. out_log_prob (device, [B, T, V] packed in lp_dtype, not
 * aliasing log_prob) receives each lane's kept rows first and zeros after them;
 * out_lengths_host [B] the kept counts. Runs on the decoder's device and stream
 * argument like wfst_decode (its scratch is the decoder's); returns after
 * synchronising the stream. Ranges as wfst_decode's, blank_id in [0, V),
 * threshold > 0 finite; both tensors device memory of the decoder's device
 * holding B * T * V elements. Errors: WFST_EINVAL, WFST_EDEVICE.
 */
int wfst_blank_skip(wfst_decoder_t d, const void *log_prob, int32_t B, int32_t T, int32_t V,
                    const int32_t *lengths_host, int32_t blank_id, float threshold, void *out_log_prob,
                    int32_t *out_lengths_host, void *stream);

/*
 * The pruned lattice of lane `lane` in the last decode (lattice mode; section 7
 * "Lattice": flat records). *n = the number of kept arcs; the first min(*n, cap)
 * records are written to out, 8 int32 each, in no particular order:
 *   {frame t, source state, destination state (the super-final state for final
 *    and redirect arcs), ilabel (-1 final, the epsilon id for an epsilon arc),
 *    arc id (num_arcs + state for the redirect's virtual arc), arc score bits
 *    (binary32 s), lane, flags (1 final arc, 2 redirect, 4 epsilon arc)}
 * A source is the token of its state at frame t, an emitting arc's destination
 * the token of its state at frame t + 1, an epsilon arc's the token of its
 * state at frame t (each epsilon arc appears once per frame). A lane with no
 * result, or whose lattice overflowed lattice_cap, has no arcs.
 * Errors: WFST_EINVAL (not lattice mode, lane outside the last decode, null),
 * WFST_EDEVICE.
 */
int wfst_lattice_records(wfst_decoder_t d, int32_t lane, int32_t *out, int64_t cap, int64_t *n);

/*
 * Counters of the last decode or stream call, summed over its lanes (n up to 17 values):
 *  [0] candidate arcs expanded on real and final steps, [1] admitted candidates,
 *  [2] distinct admitted destinations, [3] frontier tokens expanded (sum of
 *  frontier sizes), [4] epsilon arcs relaxed, [5] epsilon candidates admitted,
 *  [6] epsilon destinations claimed, [7] tokens appended or replaced by the
 *  closure, [8] winners-log entries written, [9] steps run (frame loop length),
 *  [10] largest frontier, [11] device bytes held by the decoder and its graph
 *  (the winners log as committed),
 *  [12] real (frame) steps run, summed over lanes, [13] candidates listed by
 *  the slot passes (a superset of [1]: every candidate above the running
 *  maximum minus the beam while the exact maximum was still being found),
 *  [14] winners-log address space reserved (bytes), [15] winners-log bytes
 *  committed, [16] runs of the last decode repeated after a commit (0: none).
 */
int wfst_decoder_stats(wfst_decoder_t d, int64_t *out, int32_t n);

/*
 * Device memory of a decoder (page section 6.2, wfst_decoder_mem_stats), bytes:
 *  out[0] reserved: the fixed workspace plus the winners-log address range,
 *  out[1] committed: the fixed workspace plus the winners-log memory mapped,
 *  out[2] fixed: the workspace allocated whole at creation (tokens, tables,
 *         candidate lists, records, results; not the graph),
 *  out[3] winners-log high water: the largest lane's log after the last
 *         decode or stream call (entries x 8).
 * Errors: WFST_EINVAL (null), WFST_EDEVICE.
 */
int wfst_decoder_mem_stats(wfst_decoder_t d, int64_t out[4]);

/*
 * Per-step records of lane `lane` in the last decode or stream call (steps
 * numbered from the call's first), 16 int64 each:
 *  {n, beam bits, max bits, arcs, admitted, distinct, eps arcs, eps admitted,
 *   eps distinct, eps new, eps replaced, eps passes, phase, listed, 0, 0}
 * record 0 describes the start frontier's closure (only the eps fields), record
 * t + 1 step t. phase: 0 real, 1 final, 2 redirect, 3 dead, -1 not run.
 * Writes min(steps_cap, lengths[lane] + 2) records; returns how many it wrote
 * or a negative status.
 */
int wfst_decoder_step_stats(wfst_decoder_t d, int32_t lane, int64_t *out, int32_t steps_cap);

/* Kernel ids of wfst_decoder_kernel_times, in launch order within a step. */
#define WFST_K_CLEAR        0  /* per-decode clear of records and stale recombination tables */
#define WFST_K_INIT         1  /* lane control blocks and start tokens                     */
#define WFST_K_LPMAX        2  /* max log-prob per (lane, frame) row for the bound skip    */
#define WFST_K_MAX          3  /* slot pass: exact maximum, superset admit + recombination  */
#define WFST_K_EXPAND       4  /* not launched (its work is part of WFST_K_MAX)            */
#define WFST_K_FINALIZE     5  /* exact admit, compaction, winners log, next lower bound   */
#define WFST_K_EPS_EXPAND   6  /* closure pass: relax epsilon arcs                         */
#define WFST_K_EPS_RESOLVE  7  /* not launched (its work is part of WFST_K_EPS_APPLY)      */
#define WFST_K_EPS_APPLY    8  /* closure pass: append / replace decisions and their writes */
#define WFST_K_BACKTRACK    9  /* best path (or a stream's best current token) to arcs, words */
#define WFST_K_STREAM_BEGIN 10 /* stream call: applies the per-lane plan                   */
#define WFST_K_STREAM_END  11  /* stream call: commits the chunk's last compaction        */
#define WFST_K_RECLASS     12  /* stream end: final-step class of the stream's tokens      */
#define WFST_K_LAT_RESOLVE 13  /* not launched (the next step's WFST_K_FINALIZE does it)  */
#define WFST_K_LAT_INIT    14  /* lattice with closure: backward scores to -inf           */
#define WFST_K_LAT_BACK    15  /* lattice with closure: backward pass and prune of a step */
#define WFST_K_GC_BEGIN    16  /* log compaction round: set-up and commit                 */
#define WFST_K_GC_MARK     17  /* log compaction: live entries from the frontier          */
#define WFST_K_GC_SCAN     18  /* log compaction: positions of live entries               */
#define WFST_K_GC_COMPACT  19  /* log compaction: renumbered entries into the buffer      */
#define WFST_K_GC_COMMIT   20  /* log compaction: buffer back into the log                */
#define WFST_K_GC_ROOTS    21  /* log compaction: the frontier's entries renumbered       */
#define WFST_K_GC_CLEAR    22  /* log compaction: live map and counts cleared             */
#define WFST_K_GC_END      23  /* log compaction: log end and the sealed prefix           */
#define WFST_K_LAT_EPS_BACK 24 /* lattice: a frame's epsilon arcs, fixpoint end and prune */
#define WFST_K_LAT_PRUNE   25  /* lattice: interval prune of the last 2N frames' arcs      */
#define WFST_K_LAT_EPS_ROUND 26 /* lattice: one flat relaxation round of a frame's epsilon arcs */
#define WFST_K_EPS_APPLY_EXPAND 27 /* closure: pass k's decisions and writes, then pass k + 1's relaxation */
#define WFST_K_LAT_PREP    28  /* lattice: the interval prune's arc scores, flat over lanes */
#define WFST_K_LAT_FPREP   29  /* lattice without closure: the final pass's arc scores, flat */
#define WFST_K_LAT_SWEEP   30  /* lattice without closure: backward sweep and prune per lane */
#define WFST_K_LAT_EMIT    31  /* lattice without closure: the kept arcs written out        */
#define WFST_K_COUNT       32

/*
 * Turn per-kernel timing on (enable != 0) or off. While on, each decode runs its
 * kernels as plain launches (no graph replay, as the page's sections 9 and 12
 * profile), each with a start / end hipEvent pair that its dispatch records on
 * the decode's stream, so each pair spans that kernel's execution alone.
 * Results are identical with timing on or off.
 * Errors: WFST_EINVAL, WFST_EDEVICE.
 */
int wfst_decoder_profile(wfst_decoder_t d, int32_t enable);

/*
 * Per-kernel times of the last decode, which must have run with timing on:
 * out[2*k] = total milliseconds and out[2*k + 1] = launches of kernel id k
 * (WFST_K_*), for k < min(n / 2, WFST_K_COUNT). Errors: WFST_EINVAL (null, or
 * the last decode was not profiled), WFST_EDEVICE.
 */
int wfst_decoder_kernel_times(wfst_decoder_t d, double *out, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* WFST_H */
