/*
 * CPU oracle for the WFST Viterbi beam search -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load or run this file. The decoder library never links it, and it shares no
 * code with the GPU path (no headers, helpers, tables or constants).
 *
 * It is a plain, single-threaded token-passing search written from the page
 * "GPU WFST Beam-Search Decoder" (OASR docs), section 1 "Purpose and
 * Responsibilities" (the relaxation end = score[src] + arc_weight +
 * log_prob[t][ilabel], recombination by destination, backtrack through arc ids
 * to words) and section 3 "Decoding Semantics (k2 parity)" (dynamic beam, soft
 * max_active, exact admit test, final step, allow_partial), with the epsilon
 * closure of section 5.5 and the fp32 evaluation order of section 5.3.
 * Where those sections leave a step open, the reading taken is stated at the
 * function that takes it.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (x86-64 SSE arithmetic, so
 * every float operation is one IEEE binary32 rounding; no FMA contraction).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t num_states;   /* N + 1: the last state is the super-final state */
    int32_t num_arcs;
    int32_t start;
    int32_t vocab;
    int32_t epsilon_id;   /* -1: no epsilon arcs */
    const int32_t *row_splits; /* [num_states + 1] */
    const int32_t *dest;
    const int32_t *ilabel;     /* -1 final, epsilon_id, else emitting label in [0, vocab) */
    const int32_t *olabel;     /* 0: no word */
    const float *weight;       /* log-score added to the path score */
} wo_graph;

typedef struct {
    float beam;
    int32_t min_active;
    int32_t max_active;
    int32_t allow_partial;
    int32_t eps_iterations;
    int32_t online;    /* 1: streaming (online) semantics, see wo_decode */
    int32_t partial;   /* 1: no final step; the result is the best current token */
} wo_config;

/* Per-step record written for every step the lane runs (t = 0 .. T). */
enum {
    WO_N = 0,        /* frontier size entering the step                     */
    WO_BEAM,         /* beam b_t (float bits)                               */
    WO_MAX,          /* exact maximum M_t over the step's candidates (bits) */
    WO_CUTOFF,       /* M_t - b_t (bits)                                    */
    WO_ARCS,         /* candidate arcs expanded (S_t)                       */
    WO_ADMITTED,     /* candidates with end > cutoff (C_t)                  */
    WO_DISTINCT,     /* distinct destination states among them (D_t)        */
    WO_EPS_ARCS,     /* epsilon arcs relaxed by the closure after the step  */
    WO_EPS_ADMITTED, /* of which end > cutoff                               */
    WO_EPS_DISTINCT, /* distinct destinations over the closure's passes     */
    WO_EPS_NEW,      /* tokens appended by the closure                      */
    WO_EPS_REPLACED, /* tokens replaced by the closure                      */
    WO_EPS_PASSES,   /* closure passes that had at least one source         */
    WO_N_NEXT,       /* frontier size after the step (and its closure)      */
    WO_PHASE,        /* 0 real step, 1 final step, 2 redirect, 3 dead       */
    WO_FIELDS = 16
};

typedef struct {
    float score;            /* -inf when no path */
    int32_t reached_final;
    int32_t dead;           /* 1: the lane had no candidate on a real step */
    int32_t n_arcs;         /* true path length (may exceed arcs_cap)      */
    int32_t n_words;        /* true word count                             */
    int32_t n_steps;        /* records written (may exceed steps_cap)      */
    int64_t log_entries;    /* winners-log entries the search appended      */
    int64_t start_closure[8]; /* eps arcs, admitted, distinct, new, replaced, passes, n after */
} wo_result;

/* Lattice output (page section 1 "Lattice mode", section 3 on output_beam,
 * section 7 "Lattice"): every admitted candidate of every step is a lattice arc
 * from its source token (frame t) to its destination's token (frame t + 1, or
 * the super-final state on the final step). Each record is
 * {frame, src state, dst state, ilabel (-1 final), arc id, score bits, keep, flags}
 * with the arc's own score s (weight + log-prob, one binary32 addition; a final
 * arc's weight; 0 for the redirect's virtual arc, flags 2; final arcs flags 1),
 * and vals {fwd(src), s, bwd(dst)}. keep is the output_beam prune.
 * On graphs with epsilon arcs (section 5.5: the candidate set is persisted
 * after the closure, epsilon arcs tagged) every epsilon candidate a closure
 * admitted is also a lattice arc, from its source's token to its destination's
 * token within the same frame: frame f is the frame the closure prepared
 * (0 for the start closure, t + 1 after step t), ilabel the epsilon id, s the
 * arc's weight, flags 4. An epsilon arc admitted by several passes of one
 * closure (its source improved in between) is one lattice arc. */
typedef struct {
    float output_beam;   /* finite, >= 0 */
    int64_t cap;         /* records rec / vals hold */
    int64_t n;           /* lattice arcs (true count, may exceed cap) */
    int32_t *rec;        /* [cap][8] */
    float *vals;         /* [cap][3] */
    int32_t prune_interval; /* > 0: the interval prune of section 7 every that many steps (wo_decode) */
    int64_t max_live;    /* out: most lattice arcs held at once during the search */
} wo_lattice;

/* ---- ordering key: greater = better (higher score, then smaller arc id) ---- */

/* Monotone map from binary32 to u32: a < b (as floats) iff map(a) < map(b).
 * -0.0 is first turned into +0.0 so that equal floats get equal keys. */
static uint32_t wo_float_order(float f)
{
    uint32_t u;
    if (f == 0.0f) f = 0.0f;
    memcpy(&u, &f, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static float wo_float_unorder(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* key(score, arc) = order(score) << 32 | (0xFFFFFFFF - arc); arc -1 (the start
 * token, which has no arc) gives the lowest tie rank. */
static uint64_t wo_key(float score, int32_t arc)
{
    return ((uint64_t)wo_float_order(score) << 32) | (uint64_t)(0xffffffffu - (uint32_t)arc);
}

/* ---- growable arrays ---- */

typedef struct { int32_t *state, *entry, *last; float *score; int64_t n, cap; } wo_front;
typedef struct { int32_t *prev, *arc; int64_t n, cap; } wo_log;
typedef struct { int32_t *v; int64_t n, cap; } wo_ivec;

static int wo_front_push(wo_front *f, int32_t s, float sc, int32_t e, int32_t last)
{
    if (f->n == f->cap) {
        int64_t nc = f->cap ? 2 * f->cap : 1024;
        int32_t *a = realloc(f->state, nc * 4), *b, *c;
        float *d;
        if (!a) return -1;
        f->state = a;
        if (!(b = realloc(f->entry, nc * 4))) return -1;
        f->entry = b;
        if (!(c = realloc(f->last, nc * 4))) return -1;
        f->last = c;
        if (!(d = realloc(f->score, nc * 4))) return -1;
        f->score = d;
        f->cap = nc;
    }
    f->state[f->n] = s; f->score[f->n] = sc; f->entry[f->n] = e; f->last[f->n] = last;
    f->n++;
    return 0;
}

static int64_t wo_log_push(wo_log *l, int32_t prev, int32_t arc)
{
    if (l->n == l->cap) {
        int64_t nc = l->cap ? 2 * l->cap : 4096;
        int32_t *a = realloc(l->prev, nc * 4), *b;
        if (!a) return -1;
        l->prev = a;
        if (!(b = realloc(l->arc, nc * 4))) return -1;
        l->arc = b;
        l->cap = nc;
    }
    l->prev[l->n] = prev; l->arc[l->n] = arc;
    return l->n++;
}

typedef struct { float *v; int64_t n, cap; } wo_fvec;

static int wo_fvec_push(wo_fvec *v, float x)
{
    if (v->n == v->cap) {
        int64_t nc = v->cap ? 2 * v->cap : 1024;
        float *a = realloc(v->v, nc * 4);
        if (!a) return -1;
        v->v = a; v->cap = nc;
    }
    v->v[v->n++] = x;
    return 0;
}

static int wo_ivec_push(wo_ivec *v, int32_t x)
{
    if (v->n == v->cap) {
        int64_t nc = v->cap ? 2 * v->cap : 1024;
        int32_t *a = realloc(v->v, nc * 4);
        if (!a) return -1;
        v->v = a; v->cap = nc;
    }
    v->v[v->n++] = x;
    return 0;
}

/* Arc ranges of a state: [eps arcs][emitting arcs][final arcs]. */
typedef struct { int32_t eps_b, emit_b, fin_b, end; } wo_range;

static wo_range wo_state_range(const wo_graph *g, int32_t s)
{
    wo_range r;
    int32_t a = g->row_splits[s], e = g->row_splits[s + 1];
    r.eps_b = a;
    if (g->epsilon_id >= 0)
        while (a < e && g->ilabel[a] == g->epsilon_id) a++;
    r.emit_b = a;
    while (a < e && g->ilabel[a] != -1) a++;
    r.fin_b = a;
    r.end = e;
    return r;
}

/* Shared scratch of one decode. */
typedef struct {
    int32_t *tok_of_state;  /* state -> index in the current frontier, -1 if absent */
    uint64_t *best_key;     /* state -> best candidate key this step, 0 if none     */
    int32_t *best_src;      /* state -> winners-log entry of that candidate's source */
    wo_ivec touched;        /* states with best_key != 0                            */
    /* lattice mode on epsilon graphs: the admitted epsilon arcs of each closure
     * (source token index in its frontier, arc), one entry per arc and frame */
    int lat;                /* 1: record them                                        */
    int32_t *eps_seen;      /* arc -> 1 + the frame whose closure last recorded it   */
    int32_t frame;          /* frame the running closure prepares                    */
    wo_ivec le_src, le_arc;
} wo_scratch;

/* Offer candidate (dest d, score end, arc a, source entry e) to recombination:
 * keep the greatest key per destination (section 1 "Recombination"). */
static int wo_offer(wo_scratch *sc, int32_t d, float end, int32_t a, int32_t e)
{
    uint64_t k = wo_key(end, a);
    if (sc->best_key[d] == 0) {
        if (wo_ivec_push(&sc->touched, d)) return -1;
    }
    if (k > sc->best_key[d]) {
        sc->best_key[d] = k;
        sc->best_src[d] = e;
    }
    return 0;
}

/*
 * Epsilon closure of frontier f (section 5.5 of the page: closure passes after a
 * real step, each relaxing epsilon arcs, recombining per destination, and
 * either appending a new token or improving the live one with a fresh
 * winners-log entry).
 * Readings: the pass cutoff is the frame cutoff given by the caller; pass 1
 * relaxes every token, a later pass only the tokens appended or replaced by the
 * pass before it; the candidates of a pass all use the scores the tokens had
 * when the pass began (the whole pass is relaxed before any token changes); an
 * existing token is replaced only by a strictly greater key(score, arc), where
 * its own key uses the arc that created its current entry. Stops when a pass
 * changes nothing or after eps_iterations passes.
 */
static int wo_closure(const wo_graph *g, int32_t passes_max, float cutoff, wo_front *f,
                      wo_log *lg, wo_scratch *sc, int64_t *stat /* [7] */)
{
    wo_ivec src = {0}, nxt = {0};
    int32_t *snap_s = NULL, *snap_e = NULL;
    float *snap_sc = NULL;
    int rc = -1;
    for (int64_t i = 0; i < f->n; i++)
        if (wo_ivec_push(&src, (int32_t)i)) goto out;
    for (int32_t pass = 0; pass < passes_max && src.n > 0; pass++) {
        stat[5]++;
        snap_s = realloc(snap_s, src.n * 4);
        snap_e = realloc(snap_e, src.n * 4);
        snap_sc = realloc(snap_sc, src.n * 4);
        if (!snap_s || !snap_e || !snap_sc) goto out;
        for (int64_t j = 0; j < src.n; j++) {
            int32_t i = src.v[j];
            snap_s[j] = f->state[i]; snap_sc[j] = f->score[i]; snap_e[j] = f->entry[i];
        }
        sc->touched.n = 0;
        for (int64_t j = 0; j < src.n; j++) {
            wo_range r = wo_state_range(g, snap_s[j]);
            for (int32_t a = r.eps_b; a < r.emit_b; a++) {
                float end = snap_sc[j] + g->weight[a];
                stat[0]++;
                if (end > cutoff) {
                    stat[1]++;
                    if (wo_offer(sc, g->dest[a], end, a, snap_e[j])) goto out;
                    if (sc->lat && sc->eps_seen[a] != sc->frame + 1) {
                        /* a lattice arc of this frame (once, whichever pass admits it first) */
                        sc->eps_seen[a] = sc->frame + 1;
                        if (wo_ivec_push(&sc->le_src, src.v[j]) || wo_ivec_push(&sc->le_arc, a)) goto out;
                    }
                }
            }
        }
        stat[2] += sc->touched.n;
        nxt.n = 0;
        for (int64_t j = 0; j < sc->touched.n; j++) {
            int32_t d = sc->touched.v[j];
            uint64_t k = sc->best_key[d];
            float end = wo_float_unorder((uint32_t)(k >> 32));
            int32_t a = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
            int32_t i = sc->tok_of_state[d];
            sc->best_key[d] = 0;
            if (i < 0) {
                int64_t e = wo_log_push(lg, sc->best_src[d], a);
                if (e < 0 || wo_front_push(f, d, end, (int32_t)e, a)) goto out;
                sc->tok_of_state[d] = (int32_t)(f->n - 1);
                if (wo_ivec_push(&nxt, (int32_t)(f->n - 1))) goto out;
                stat[3]++;
            } else if (k > wo_key(f->score[i], f->last[i])) {
                int64_t e = wo_log_push(lg, sc->best_src[d], a);
                if (e < 0) goto out;
                f->score[i] = end; f->entry[i] = (int32_t)e; f->last[i] = a;
                if (wo_ivec_push(&nxt, i)) goto out;
                stat[4]++;
            }
        }
        sc->touched.n = 0;
        { wo_ivec t = src; src = nxt; nxt = t; }
    }
    stat[6] = f->n;
    rc = 0;
out:
    free(src.v); free(nxt.v); free(snap_s); free(snap_e); free(snap_sc);
    return rc;
}

/*
 * Decode one utterance: lp points at its log-prob rows (row t at lp + t*lp_stride,
 * V floats each), T is its length. Returns 0, or -1 on allocation failure,
 * -2 on invalid arguments.
 *
 * Per step t = 0..T (t == T is the final step):
 *  beam (section 3 "Dynamic beam"): final step b = 1e10; otherwise with
 *    min_active raised to max(min_active, max_active/2) when T - t <= 5 (the
 *    reading of "the last ~5 frames"), b = min(b', beam)*0.8 when n > max_active,
 *    b = max(b', beam)*1.25 when n < min_active, else b = 0.8*b' + 0.2*beam, where
 *    b' is the previous step's b (beam before step 0) and n the frontier size.
 *    All in binary32, each operation rounded.
 *  candidates: every emitting arc (final arc on the final step) of every token;
 *    end = (score + weight) + lp[t][ilabel] in that order (section 5.3), or
 *    score + weight on the final step.
 *  exact maximum M over all candidates; admit end > M - b (strict, section 3
 *    "Admit test"); keep per destination the greatest key(end, arc).
 *  winners become the next frontier, each with a winners-log entry
 *    {source entry, arc}; on epsilon graphs the closure follows every real step
 *    (and runs once on the start frontier with cutoff 0 - beam).
 * A real step with no candidate, or an empty frontier, ends the lane (dead). A
 * final step with no candidate redirects when allow_partial is set: each token
 * is offered with a virtual arc of weight 0 and id num_arcs + state, and the
 * best key wins (reached_final = 0, the virtual arc is not on the path).
 *
 * Streaming (section 3, last paragraph, and section 8 "Streaming Lifecycle"):
 * with cfg->online the utterance length is unknown while frames arrive (T is
 * unbounded until the caller ends the stream), so the "last ~5 frames" raise of
 * min_active never applies; ending the stream at T runs the same final step.
 * Chunk boundaries are invisible to the search, so online decoding of T frames
 * in any chunking is this one call. With cfg->partial the search stops after
 * the T real steps (and their closures) without a final step, and the result is
 * the partial hypothesis of section 8: the path of the best token of the current
 * frontier. Reading: best = greatest key(score, arc that gave the token its
 * current score), the same order as recombination (higher score, then smaller
 * arc id; the start token's arc -1 ranks lowest); reached_final = 0.
 */
int wo_decode(const wo_graph *g, const wo_config *cfg, const float *lp, int32_t T,
              int64_t lp_stride, int32_t *arcs, int32_t arcs_cap, int32_t *words,
              int32_t words_cap, int64_t *steps, int32_t steps_cap, wo_result *res,
              wo_lattice *lat)
{
    wo_front cur = {0}, nxt = {0};
    wo_log lg = {0};
    wo_scratch sc = {0};
    /* lattice: tokens of every frame (state, score), arcs of every step
     * (source token index in its frame, arc id, arc score), offsets by step */
    wo_ivec lt_state = {0}, la_src = {0}, la_arc = {0};
    wo_fvec lt_score = {0}, la_s = {0};
    int64_t *lt_off = NULL, *la_off = NULL;
    int64_t *le_beg = NULL, *le_end = NULL;   /* epsilon lattice arcs of frame f: [le_beg[f], le_end[f]) */
    int32_t *pmap = NULL;                     /* interval prune: state -> token index of one frame */
    int32_t lat_steps = 0;
    int rc = -1;
    int32_t final_entry = -1;
    int have_path = 0;
    float b_prev = cfg->beam;

    memset(res, 0, sizeof(*res));
    res->score = -INFINITY;
    if (!g || !cfg || T < 0 || (T > 0 && !lp)) return -2;
    /* lattice mode: not with partial results; on epsilon graphs every epsilon
     * weight must be <= 0 (reading: then a token's best continuation inside its
     * frame exists, since no epsilon cycle can raise it) */
    if (lat && (cfg->partial || !(lat->output_beam >= 0.0f) || isinf(lat->output_beam))) return -2;
    if (lat && g->epsilon_id >= 0 && cfg->eps_iterations > 0)
        for (int32_t a = 0; a < g->num_arcs; a++)
            if (g->ilabel[a] == g->epsilon_id && g->weight[a] > 0.0f) return -2;
    if (lat) {
        lat->n = 0;
        lt_off = malloc(((size_t)T + 3) * 8);
        la_off = malloc(((size_t)T + 3) * 8);
        le_beg = calloc((size_t)T + 3, 8);
        le_end = calloc((size_t)T + 3, 8);
        if (!lt_off || !la_off || !le_beg || !le_end) goto out;
        if (g->epsilon_id >= 0 && cfg->eps_iterations > 0) {
            sc.lat = 1;
            sc.eps_seen = calloc((size_t)(g->num_arcs > 0 ? g->num_arcs : 1), 4);
            if (!sc.eps_seen) goto out;
        }
        lat->max_live = 0;
        if (lat->prune_interval < 0) { rc = -2; goto out; }
        if (lat->prune_interval > 0) {
            pmap = malloc((size_t)g->num_states * 4);
            if (!pmap) goto out;
            for (int32_t st = 0; st < g->num_states; st++) pmap[st] = -1;
        }
    }
    sc.tok_of_state = malloc((size_t)g->num_states * 4);
    sc.best_key = calloc((size_t)g->num_states, 8);
    sc.best_src = malloc((size_t)g->num_states * 4);
    if (!sc.tok_of_state || !sc.best_key || !sc.best_src) goto out;
    for (int32_t s = 0; s < g->num_states; s++) sc.tok_of_state[s] = -1;

    if (wo_front_push(&cur, g->start, 0.0f, -1, -1)) goto out;
    sc.tok_of_state[g->start] = 0;
    if (g->epsilon_id >= 0 && cfg->eps_iterations > 0) {
        float cut0 = 0.0f - cfg->beam;
        sc.frame = 0;
        if (lat) le_beg[0] = sc.le_src.n;
        if (wo_closure(g, cfg->eps_iterations, cut0, &cur, &lg, &sc, res->start_closure)) goto out;
        if (lat) le_end[0] = sc.le_src.n;
    }

    for (int32_t t = 0; t <= T; t++) {
        int is_final = (t == T);
        int64_t n = cur.n;
        if (is_final && cfg->partial) {
            /* partial hypothesis: the best token of the current frontier */
            int64_t bi = -1;
            uint64_t bk = 0;
            for (int64_t i = 0; i < n; i++) {
                uint64_t k = wo_key(cur.score[i], cur.last[i]);
                if (bi < 0 || k > bk) { bk = k; bi = i; }
            }
            if (bi >= 0) {
                res->score = cur.score[bi];
                res->reached_final = 0;
                final_entry = cur.entry[bi];
                have_path = 1;
            } else {
                res->dead = 1;
            }
            break;
        }
        int64_t rec[WO_FIELDS];
        float b, M = -INFINITY, cutoff;
        int64_t S = 0, C = 0;
        memset(rec, 0, sizeof(rec));
        rec[WO_N] = n;
        rec[WO_PHASE] = is_final ? 1 : 0;
        if (lat) {
            lt_off[t] = lt_state.n;
            la_off[t] = la_src.n;
            lat_steps = t + 1;
            for (int64_t i = 0; i < n; i++)
                if (wo_ivec_push(&lt_state, cur.state[i]) || wo_fvec_push(&lt_score, cur.score[i])) goto out;
        }
        if (n == 0) {
            res->dead = 1;
            rec[WO_PHASE] = 3;
            if (res->n_steps < steps_cap) memcpy(steps + (int64_t)res->n_steps * WO_FIELDS, rec, sizeof(rec));
            res->n_steps++;
            break;
        }
        if (is_final) {
            b = 1e10f;
        } else {
            int32_t mina = cfg->min_active;
            if (!cfg->online && T - t <= 5 && cfg->max_active / 2 > mina) mina = cfg->max_active / 2;
            if (n > cfg->max_active) {
                b = (b_prev < cfg->beam ? b_prev : cfg->beam) * 0.8f;
            } else if (n < mina) {
                b = (b_prev > cfg->beam ? b_prev : cfg->beam) * 1.25f;
            } else {
                float x = 0.8f * b_prev;
                float y = 0.2f * cfg->beam;
                b = x + y;
            }
            b_prev = b;
        }
        { uint32_t u; memcpy(&u, &b, 4); rec[WO_BEAM] = u; }

        /* pass 1: the exact maximum over every candidate of the step */
        for (int64_t i = 0; i < n; i++) {
            wo_range r = wo_state_range(g, cur.state[i]);
            int32_t a0 = is_final ? r.fin_b : r.emit_b, a1 = is_final ? r.end : r.fin_b;
            const float *row = is_final ? NULL : lp + (int64_t)t * lp_stride;
            for (int32_t a = a0; a < a1; a++) {
                float end = cur.score[i] + g->weight[a];
                if (!is_final) end = end + row[g->ilabel[a]];
                if (S == 0 || end > M) M = end;
                S++;
            }
        }
        rec[WO_ARCS] = S;
        if (S == 0) {
            if (is_final && cfg->allow_partial) {
                /* redirect: best token by key(score + 0, num_arcs + state) */
                uint64_t bk = 0;
                int64_t bi = -1;
                for (int64_t i = 0; i < n; i++) {
                    float end = cur.score[i] + 0.0f;
                    uint64_t k = wo_key(end, (int32_t)((uint32_t)g->num_arcs + (uint32_t)cur.state[i]));
                    if (bi < 0 || k > bk) { bk = k; bi = i; }
                }
                res->score = cur.score[bi] + 0.0f;
                res->reached_final = 0;
                final_entry = cur.entry[bi];
                have_path = 1;
                rec[WO_PHASE] = 2;
                if (lat && (wo_ivec_push(&la_src, (int32_t)bi) ||
                            wo_ivec_push(&la_arc, (int32_t)((uint32_t)g->num_arcs + (uint32_t)cur.state[bi])) ||
                            wo_fvec_push(&la_s, 0.0f))) goto out;
            } else if (!is_final) {
                res->dead = 1;
                rec[WO_PHASE] = 3;
            }
            if (res->n_steps < steps_cap) memcpy(steps + (int64_t)res->n_steps * WO_FIELDS, rec, sizeof(rec));
            res->n_steps++;
            break;
        }
        cutoff = M - b;
        { uint32_t u; memcpy(&u, &M, 4); rec[WO_MAX] = u; memcpy(&u, &cutoff, 4); rec[WO_CUTOFF] = u; }

        /* pass 2: admit and recombine by destination */
        sc.touched.n = 0;
        for (int64_t i = 0; i < n; i++) {
            wo_range r = wo_state_range(g, cur.state[i]);
            int32_t a0 = is_final ? r.fin_b : r.emit_b, a1 = is_final ? r.end : r.fin_b;
            const float *row = is_final ? NULL : lp + (int64_t)t * lp_stride;
            for (int32_t a = a0; a < a1; a++) {
                float end = cur.score[i] + g->weight[a];
                if (!is_final) end = end + row[g->ilabel[a]];
                if (end > cutoff) {
                    C++;
                    if (wo_offer(&sc, g->dest[a], end, a, cur.entry[i])) goto out;
                    if (lat) {
                        /* the arc's own score: weight + log-prob (final: weight) */
                        float sa = is_final ? g->weight[a] : g->weight[a] + row[g->ilabel[a]];
                        if (wo_ivec_push(&la_src, (int32_t)i) || wo_ivec_push(&la_arc, a) ||
                            wo_fvec_push(&la_s, sa)) goto out;
                    }
                }
            }
        }
        rec[WO_ADMITTED] = C;
        rec[WO_DISTINCT] = sc.touched.n;

        /* next frontier: one token per winning destination */
        for (int64_t i = 0; i < n; i++) sc.tok_of_state[cur.state[i]] = -1;
        nxt.n = 0;
        for (int64_t j = 0; j < sc.touched.n; j++) {
            int32_t d = sc.touched.v[j];
            uint64_t k = sc.best_key[d];
            float end = wo_float_unorder((uint32_t)(k >> 32));
            int32_t a = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
            int64_t e = wo_log_push(&lg, sc.best_src[d], a);
            sc.best_key[d] = 0;
            if (e < 0 || wo_front_push(&nxt, d, end, (int32_t)e, a)) goto out;
            sc.tok_of_state[d] = (int32_t)(nxt.n - 1);
        }
        sc.touched.n = 0;
        { wo_front tmp = cur; cur = nxt; nxt = tmp; }

        if (is_final) {
            /* every final arc enters the super-final state, so cur holds at most one token */
            if (cur.n > 0) {
                res->score = cur.score[0];
                res->reached_final = 1;
                final_entry = cur.entry[0];
                have_path = 1;
            }
            rec[WO_N_NEXT] = cur.n;
            if (res->n_steps < steps_cap) memcpy(steps + (int64_t)res->n_steps * WO_FIELDS, rec, sizeof(rec));
            res->n_steps++;
            break;
        }
        if (g->epsilon_id >= 0 && cfg->eps_iterations > 0) {
            int64_t st[8] = {0};
            sc.frame = t + 1;
            if (lat) le_beg[t + 1] = sc.le_src.n;
            if (wo_closure(g, cfg->eps_iterations, cutoff, &cur, &lg, &sc, st)) goto out;
            if (lat) le_end[t + 1] = sc.le_src.n;
            rec[WO_EPS_ARCS] = st[0]; rec[WO_EPS_ADMITTED] = st[1]; rec[WO_EPS_DISTINCT] = st[2];
            rec[WO_EPS_NEW] = st[3]; rec[WO_EPS_REPLACED] = st[4]; rec[WO_EPS_PASSES] = st[5];
        }
        rec[WO_N_NEXT] = cur.n;
        if (res->n_steps < steps_cap) memcpy(steps + (int64_t)res->n_steps * WO_FIELDS, rec, sizeof(rec));
        res->n_steps++;
        if (lat && la_src.n + sc.le_src.n > lat->max_live) lat->max_live = la_src.n + sc.le_src.n;

        /*
         * Interval prune (section 7: lat_prune_interval = N, a window-loose
         * prune that bounds the lattice while the exact final pass stays as it
         * is). Reading: after every N-th real step that is not the last one,
         * with F = t + 1 the frontier's frame and W = max(0, F - 2N), backward
         * scores over frames W .. F - 1 are computed as in the final pass but
         * from bwd(u) = -fwd(u) for every frontier token u (no complete path
         * through u can score more than the final best, so fwd(u) + bwd(u) is
         * at most best - fwd(u) + fwd(u)); the arcs of steps W .. F - 1 and the
         * epsilon arcs of frames W .. F - 1 with (fwd(src) + s) + bwd(dst) <
         * 0 - output_beam are removed: the final test, which subtracts the
         * same output beam from the best, could not keep them (exactly so in
         * exact arithmetic). Survivors keep their order.
         */
        if (lat && lat->prune_interval > 0 && (t + 1) % lat->prune_interval == 0 && t + 1 < T) {
            const int32_t F = t + 1;
            const int32_t W = F - 2 * lat->prune_interval > 0 ? F - 2 * lat->prune_interval : 0;
            const float thr_loose = 0.0f - lat->output_beam;
            const int64_t ea0 = la_off[W], ea1 = la_src.n;
            const int64_t xa0 = sc.lat ? le_beg[W] : 0, xa1 = sc.lat ? sc.le_src.n : 0;
            uint8_t *keep_e = malloc((size_t)(ea1 - ea0 + 1));
            uint8_t *keep_x = malloc((size_t)(xa1 - xa0 + 1));
            float *bnext = malloc((size_t)(cur.n > 0 ? cur.n : 1) * 4);
            if (!keep_e || !keep_x || !bnext) { free(keep_e); free(keep_x); free(bnext); goto out; }
            memset(keep_e, 1, (size_t)(ea1 - ea0 + 1));
            memset(keep_x, 1, (size_t)(xa1 - xa0 + 1));
            for (int64_t i = 0; i < cur.n; i++) bnext[i] = -cur.score[i];
            for (int32_t f = F - 1; f >= W; f--) {
                const int64_t fa = lt_off[f], fb = (f + 1 <= t) ? lt_off[f + 1] : lt_state.n;
                const int64_t nf = fb - fa;
                const int64_t k0 = la_off[f], k1 = (f + 1 <= t) ? la_off[f + 1] : la_src.n;
                float *b = malloc((size_t)(nf > 0 ? nf : 1) * 4);
                if (!b) { free(keep_e); free(keep_x); free(bnext); goto out; }
                for (int64_t i = 0; i < nf; i++) b[i] = -INFINITY;
                /* destinations: frame f + 1's tokens (the frontier's own map at F) */
                if (f + 1 < F)
                    for (int64_t j = lt_off[f + 1]; j < ((f + 2 <= t) ? lt_off[f + 2] : lt_state.n); j++)
                        pmap[lt_state.v[j]] = (int32_t)(j - lt_off[f + 1]);
                for (int64_t k = k0; k < k1; k++) {
                    const int32_t i = la_src.v[k], a = la_arc.v[k];
                    const float sa = la_s.v[k];
                    const float bd = bnext[f + 1 < F ? pmap[g->dest[a]] : sc.tok_of_state[g->dest[a]]];
                    const float v = sa + bd;
                    if (v > b[i]) b[i] = v;
                    keep_e[k - ea0] = ((lt_score.v[fa + i] + sa) + bd) >= thr_loose;
                }
                if (f + 1 < F)
                    for (int64_t j = lt_off[f + 1]; j < ((f + 2 <= t) ? lt_off[f + 2] : lt_state.n); j++)
                        pmap[lt_state.v[j]] = -1;
                if (sc.lat && le_end[f] > le_beg[f]) {
                    for (int64_t j = fa; j < fb; j++) pmap[lt_state.v[j]] = (int32_t)(j - fa);
                    for (int changed = 1; changed;) {
                        changed = 0;
                        for (int64_t k = le_beg[f]; k < le_end[f]; k++) {
                            const int32_t i = sc.le_src.v[k], a = sc.le_arc.v[k];
                            const float v = g->weight[a] + b[pmap[g->dest[a]]];
                            if (v > b[i]) { b[i] = v; changed = 1; }
                        }
                    }
                    for (int64_t k = le_beg[f]; k < le_end[f]; k++) {
                        const int32_t i = sc.le_src.v[k], a = sc.le_arc.v[k];
                        keep_x[k - xa0] = ((lt_score.v[fa + i] + g->weight[a]) + b[pmap[g->dest[a]]]) >= thr_loose;
                    }
                    for (int64_t j = fa; j < fb; j++) pmap[lt_state.v[j]] = -1;
                }
                free(bnext);
                bnext = b;
            }
            free(bnext);
            /* compaction: the steps' own arcs, then the epsilon arcs (frame F's
             * all stay: its closure belongs to the next window) */
            {
                int64_t o = ea0;
                for (int32_t f = W; f < F; f++) {
                    const int64_t k0 = la_off[f], k1 = (f + 1 <= t) ? la_off[f + 1] : ea1;
                    la_off[f] = o;
                    for (int64_t k = k0; k < k1; k++)
                        if (keep_e[k - ea0]) {
                            la_src.v[o] = la_src.v[k]; la_arc.v[o] = la_arc.v[k]; la_s.v[o] = la_s.v[k];
                            o++;
                        }
                }
                la_src.n = la_arc.n = la_s.n = o;
            }
            if (sc.lat) {
                int64_t o = xa0;
                for (int32_t f = W; f <= F; f++) {
                    const int64_t k0 = le_beg[f], k1 = le_end[f];
                    le_beg[f] = o;
                    for (int64_t k = k0; k < k1; k++)
                        if (f == F || keep_x[k - xa0]) {
                            sc.le_src.v[o] = sc.le_src.v[k]; sc.le_arc.v[o] = sc.le_arc.v[k];
                            o++;
                        }
                    le_end[f] = o;
                }
                sc.le_src.n = sc.le_arc.n = o;
            }
            free(keep_e);
            free(keep_x);
        }
    }
    if (lat && la_src.n + sc.le_src.n > lat->max_live) lat->max_live = la_src.n + sc.le_src.n;

    /*
     * Lattice backward pass and output_beam prune (section 3: forward[src] + arc +
     * backward[dst] >= best - output_beam; section 1 "Lattice mode"). Readings:
     * bwd(super-final) = 0; bwd(token) = max over the token's lattice arcs of
     * s + bwd(dst), steps from the last back to the first (one binary32 addition
     * each; -inf without arcs); fwd(token) = its search score; an arc is kept iff
     * (fwd(src) + s) + bwd(dst) >= best - output_beam, in that order, with best
     * the lane's result score. Only lanes with a result have a lattice.
     */
    if (lat && have_path && lat_steps > 0) {
        float *bnext = NULL, *bcur = NULL;
        const float thresh = res->score - lat->output_beam;
        lt_off[lat_steps] = lt_state.n;
        la_off[lat_steps] = la_src.n;
        for (int32_t t = lat_steps - 1; t >= 0; t--) {
            const int64_t t0 = lt_off[t], nt = lt_off[t + 1] - t0;
            const int last = (t == lat_steps - 1);
            float *b = malloc((size_t)(nt > 0 ? nt : 1) * 4);
            if (!b) { free(bnext); goto out; }
            for (int64_t i = 0; i < nt; i++) b[i] = -INFINITY;
            /* state -> token index of frame t + 1 (the destinations) */
            if (!last)
                for (int64_t j = lt_off[t + 1]; j < lt_off[t + 2]; j++)
                    sc.tok_of_state[lt_state.v[j]] = (int32_t)(j - lt_off[t + 1]);
            for (int64_t k = la_off[t]; k < la_off[t + 1]; k++) {
                const int32_t i = la_src.v[k], a = la_arc.v[k];
                const int redirect = a >= g->num_arcs;
                const float sa = la_s.v[k];
                float bd = 0.0f;
                if (!last) bd = bnext[sc.tok_of_state[g->dest[a]]];
                const float v = sa + bd;
                if (v > b[i]) b[i] = v;
                const float fwd = lt_score.v[t0 + i];
                const float thr = (fwd + sa) + bd;
                if (lat->n < lat->cap) {
                    int32_t *r = lat->rec + lat->n * 8;
                    uint32_t u;
                    memcpy(&u, &sa, 4);
                    r[0] = t;
                    r[1] = lt_state.v[t0 + i];
                    r[2] = redirect ? g->num_states - 1 : g->dest[a];
                    r[3] = (redirect || last) ? -1 : g->ilabel[a];
                    r[4] = a;
                    r[5] = (int32_t)u;
                    r[6] = thr >= thresh ? 1 : 0;
                    r[7] = redirect ? 2 : (last ? 1 : 0);
                    lat->vals[lat->n * 3 + 0] = fwd;
                    lat->vals[lat->n * 3 + 1] = sa;
                    lat->vals[lat->n * 3 + 2] = bd;
                }
                lat->n++;
            }
            if (!last)
                for (int64_t j = lt_off[t + 1]; j < lt_off[t + 2]; j++) sc.tok_of_state[lt_state.v[j]] = -1;
            /*
             * Epsilon arcs of frame t (reading): bwd(token) also takes the best of
             * w + bwd(dst) over its epsilon arcs, whose destinations lie in the
             * same frame, so frame t's scores are the least fixpoint of those
             * relaxations on top of the step's own arcs: relaxed until nothing
             * changes (every epsilon weight is <= 0, so this ends, and the result
             * is the best right-folded continuation whatever the order). Then the
             * same keep test, with fwd(src) the source token's score after the
             * closure and s the arc's weight.
             */
            if (le_end[t] > le_beg[t]) {
                for (int64_t j = t0; j < t0 + nt; j++) sc.tok_of_state[lt_state.v[j]] = (int32_t)(j - t0);
                for (int changed = 1; changed;) {
                    changed = 0;
                    for (int64_t k = le_beg[t]; k < le_end[t]; k++) {
                        const int32_t i = sc.le_src.v[k], a = sc.le_arc.v[k];
                        const float v = g->weight[a] + b[sc.tok_of_state[g->dest[a]]];
                        if (v > b[i]) { b[i] = v; changed = 1; }
                    }
                }
                for (int64_t k = le_beg[t]; k < le_end[t]; k++) {
                    const int32_t i = sc.le_src.v[k], a = sc.le_arc.v[k];
                    const float sa = g->weight[a];
                    const float bd = b[sc.tok_of_state[g->dest[a]]];
                    const float fwd = lt_score.v[t0 + i];
                    const float thr = (fwd + sa) + bd;
                    if (lat->n < lat->cap) {
                        int32_t *r = lat->rec + lat->n * 8;
                        uint32_t u;
                        memcpy(&u, &sa, 4);
                        r[0] = t;
                        r[1] = lt_state.v[t0 + i];
                        r[2] = g->dest[a];
                        r[3] = g->epsilon_id;
                        r[4] = a;
                        r[5] = (int32_t)u;
                        r[6] = thr >= thresh ? 1 : 0;
                        r[7] = 4;
                        lat->vals[lat->n * 3 + 0] = fwd;
                        lat->vals[lat->n * 3 + 1] = sa;
                        lat->vals[lat->n * 3 + 2] = bd;
                    }
                    lat->n++;
                }
                for (int64_t j = t0; j < t0 + nt; j++) sc.tok_of_state[lt_state.v[j]] = -1;
            }
            free(bnext);
            bnext = b;
            (void)bcur;
        }
        free(bnext);
    }

    /* backtrack: entry -> prev to -1, collected newest first, written oldest first */
    if (have_path) {
        int32_t len = 0, nw = 0;
        for (int32_t e = final_entry; e >= 0; e = lg.prev[e]) len++;
        {
            int32_t k = len;
            for (int32_t e = final_entry; e >= 0; e = lg.prev[e]) {
                k--;
                if (k < arcs_cap) arcs[k] = lg.arc[e];
            }
        }
        /* words: the non-zero olabels in path order; needs the whole path */
        {
            int32_t *tmp = malloc((size_t)(len > 0 ? len : 1) * 4);
            int32_t k = len;
            if (!tmp) goto out;
            for (int32_t e = final_entry; e >= 0; e = lg.prev[e]) tmp[--k] = lg.arc[e];
            for (int32_t i = 0; i < len; i++) {
                int32_t w = g->olabel[tmp[i]];
                if (w != 0) {
                    if (nw < words_cap) words[nw] = w;
                    nw++;
                }
            }
            free(tmp);
        }
        res->n_arcs = len;
        res->n_words = nw;
    }
    res->log_entries = lg.n;
    rc = 0;
out:
    free(cur.state); free(cur.entry); free(cur.last); free(cur.score);
    free(nxt.state); free(nxt.entry); free(nxt.last); free(nxt.score);
    free(lg.prev); free(lg.arc);
    free(sc.tok_of_state); free(sc.best_key); free(sc.best_src); free(sc.touched.v);
    free(lt_state.v); free(la_src.v); free(la_arc.v); free(lt_score.v); free(la_s.v);
    free(lt_off); free(la_off); free(le_beg); free(le_end);
    free(sc.eps_seen); free(sc.le_src.v); free(sc.le_arc.v); free(pmap);
    return rc;
}

int wo_fields(void) { return WO_FIELDS; }
