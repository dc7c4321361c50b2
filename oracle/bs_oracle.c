/*
 * bs_oracle.c -- plain, slow, scalar CPU oracle for the BF16 rANS container.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product decode path
 * never calls it, and it shares no code, header, table or helper with the HIP
 * library: everything here is written out again from the format definition.
 *
 * What is computed, and where it comes from:
 *   - Each BF16 word is split into its exact fields [sign:1 | exponent:8 |
 *     fraction:7]; the joint (sign, exponent) symbol is coded with a per-tensor
 *     rANS model; once decoded it selects the distribution used for the 7-bit
 *     fraction; the decoder recombines the fields bitwise.  Non-BF16 spans are
 *     kept verbatim in a residual.
 *     [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec paragraph after the
 *      metrics table]
 *   - Every tensor carries a hash checked at decompression (sha256 here).
 *     [Gemma 2 9B Instruct -- Lossless Compressed card, "What lossless means";
 *      NVLC card, SHA256SUMS verification block]
 *   - Everything else (state width, renormalisation unit, table precisions,
 *     the quantisation rule, the choice of coded fraction contexts, the
 *     lane/chunk interleave and the byte layout) is not given by the pages.
 *     It is this container's own definition; the readings are listed in the
 *     design notes of the repository.
 *
 * The rANS coder follows Duda's range variant of asymmetric numeral systems:
 *   encode  x' = floor(x / q) * 2^M + (x mod q) + cum
 *   decode  slot = x mod 2^M, sym = the symbol with cum <= slot < cum + q,
 *           x = q * floor(x / 2^M) + slot - cum
 * with a 32-bit state kept in [2^16, 2^32) by 16-bit renormalisation words.
 *
 * Two record layouts (both this container's own definitions):
 *   layout 1 (container version 1): per weight, s is coded with the s-table
 *     and then the whole 7-bit fraction f with the table s selects; each of
 *     the two symbols is followed by a renormalisation check.
 *   layout 2 (container version 2): per weight, s (precision M_s) and the
 *     fraction's high three bits h = f >> 4 (precision M_h = 16 - M_s, with
 *     the table s selects) are coded back to back and followed by a single
 *     renormalisation check: the two steps consume at most 16 bits of the
 *     state, so one 16-bit word always restores it.  The low four bits
 *     l = f & 15 are stored verbatim in a fixed-width plane of the chunk.
 *     The fraction's distribution given s is thus P(h | s) * 2^-4.  An
 *     exponent without a coded h table of its own shares the table (flat or
 *     coded) that codes its h counts in the fewest bits (bso_share_hroutes).
 *   layout 3 (container version 3): as layout 2, except that s and h are
 *     coded as one joint symbol t = 8 s + h with a single per-tensor table
 *     of precision M_t = 13 (the normaliser applied to the joint counts):
 *     one coding step and one renormalisation check per weight.  The joint
 *     table holds P(s) P(h | s) as counted, so every s has its own h
 *     distribution.  A lane's last group codes s alone (the s-table, M_s),
 *     with its h values in the start state, and the low four bits sit in
 *     the plane, both as in layout 2.
 *
 * Parity pins live in tests/test_oracle_*.py (hand-computed coder states,
 * a bit-stack reduction, brute force, normaliser invariants, round trips).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BSO_L          65536u          /* lower end of the state interval */
#define BSO_MAGIC      "BF16RANS"
#define BSO_VERSION    1u              /* containers whose BF16 records use layout 1 */
#define BSO_VERSION2   2u              /* containers with layout-2 BF16 records */
#define BSO_VERSION3   3u              /* containers with layout-3 BF16 records */
#define BSO_MT         13u             /* precision of the joint (s, h) table of layout 3 */
#define BSO_MAX_HTABLES 31u            /* coded h tables per layout-2 record */
#define BSO_HDR_BYTES  64u
#define BSO_DIR_BYTES  96u
#define BSO_KIND_BF16  1u
#define BSO_KIND_RAW   2u
#define BSO_MAX_TABLES 6u
#define BSO_MAX_SYMS   256u            /* more occupied (sign,exp) symbols -> stored RAW */
#define BSO_CANDIDATES 64u
#define BSO_OUT_ALIGN  256u

/* error codes (negative), same meaning as the names say */
#define BSO_OK       0
#define BSO_EINVAL  -1
#define BSO_EFORMAT -2
#define BSO_EVERSION -3
#define BSO_ENOSPACE -4
#define BSO_ENOMEM  -5
#define BSO_ECORRUPT -7

/* ------------------------------------------------------------------------ */
/* little-endian helpers (explicit byte order, no type punning)              */
/* ------------------------------------------------------------------------ */
static void put16(uint8_t* p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint32_t get16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get32(const uint8_t* p) { uint32_t v = 0; for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i); return v; }
static uint64_t get64(const uint8_t* p) { uint64_t v = 0; for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i); return v; }
static uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

/* ------------------------------------------------------------------------ */
/* Field split and recombination                                             */
/* [NVLC card, codec paragraph: sign:1 | exponent:8 | fraction:7]            */
/* The joint symbol is s = sign*256 + exponent, i.e. the top 9 bits.         */
/* ------------------------------------------------------------------------ */
uint32_t bso_symbol_s(uint16_t w) { return ((uint32_t)w >> 15) * 256u + (((uint32_t)w >> 7) & 0xFFu); }
uint32_t bso_symbol_f(uint16_t w) { return (uint32_t)w & 0x7Fu; }
uint16_t bso_combine(uint32_t s, uint32_t f) {
    uint32_t sign = s / 256u, expo = s % 256u;
    return (uint16_t)((sign << 15) | (expo << 7) | f);
}

/* ------------------------------------------------------------------------ */
/* Histogram of the two fields: cs[s] and cf[s][f] (512 x 128, row major).    */
/* [NVLC card, codec paragraph: the model is per tensor]                      */
/* ------------------------------------------------------------------------ */
void bso_histogram(const uint16_t* w, uint64_t n, uint64_t* cs, uint64_t* cf) {
    memset(cs, 0, 512 * sizeof(uint64_t));
    memset(cf, 0, 512 * 128 * sizeof(uint64_t));
    for (uint64_t i = 0; i < n; i++) {
        uint32_t s = bso_symbol_s(w[i]);
        uint32_t f = bso_symbol_f(w[i]);
        cs[s] += 1;
        cf[s * 128 + f] += 1;
    }
}

/* ------------------------------------------------------------------------ */
/* Quantise counts c[0..A) to frequencies q summing to 2^M (integer only).   */
/* Container rule (the pages give none):                                     */
/*   q_i = 0 if c_i = 0, else max(1, floor(c_i 2^M / n));                    */
/*   while the sum is short, add 1 to occupied symbols in order of the       */
/*   remainder (c_i 2^M mod n) descending, lower index first on ties,        */
/*   cycling through that order;                                             */
/*   while the sum is over, take 1 from the symbol with the largest q (>1),  */
/*   lower index first on ties.                                              */
/* Returns 0, or BSO_EINVAL when nothing is occupied or 2^M is too small.    */
/* ------------------------------------------------------------------------ */
int bso_normalise(const uint64_t* c, uint32_t A, uint32_t M, uint32_t* q) {
    uint64_t n = 0, occupied = 0;
    for (uint32_t i = 0; i < A; i++) { n += c[i]; if (c[i]) occupied++; }
    if (n == 0 || occupied > ((uint64_t)1 << M)) return BSO_EINVAL;
    const unsigned __int128 total = (unsigned __int128)1 << M;
    int64_t sum = 0;
    for (uint32_t i = 0; i < A; i++) {
        if (c[i] == 0) { q[i] = 0; continue; }
        uint64_t v = (uint64_t)(((unsigned __int128)c[i] * total) / n);
        q[i] = (uint32_t)(v < 1 ? 1 : v);
        sum += q[i];
    }
    int64_t d = ((int64_t)1 << M) - sum;
    if (d > 0) {
        /* order occupied symbols by remainder descending, index ascending:
           a plain selection sort, written for clarity, not speed */
        uint32_t* order = (uint32_t*)malloc(sizeof(uint32_t) * occupied);
        uint64_t* rem = (uint64_t*)malloc(sizeof(uint64_t) * A);
        if (!order || !rem) { free(order); free(rem); return BSO_ENOMEM; }
        uint64_t k = 0;
        for (uint32_t i = 0; i < A; i++) {
            if (!c[i]) continue;
            rem[i] = (uint64_t)(((unsigned __int128)c[i] * total) % n);
            order[k++] = i;
        }
        for (uint64_t a = 0; a < k; a++) {
            uint64_t best = a;
            for (uint64_t b = a + 1; b < k; b++) {
                uint32_t ib = order[b], ibest = order[best];
                if (rem[ib] > rem[ibest] || (rem[ib] == rem[ibest] && ib < ibest)) best = b;
            }
            uint32_t t = order[a]; order[a] = order[best]; order[best] = t;
        }
        for (int64_t j = 0; j < d; j++) q[order[(uint64_t)j % k]] += 1;
        free(order); free(rem);
    }
    while (d < 0) {
        uint32_t best = A;
        for (uint32_t i = 0; i < A; i++) {
            if (q[i] > 1 && (best == A || q[i] > q[best])) best = i;
        }
        if (best == A) return BSO_EINVAL; /* unreachable when occupied <= 2^M */
        q[best] -= 1;
        d += 1;
    }
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* Choice of the coded fraction contexts (container rule, integer only).     */
/* [NVLC card, codec paragraph: the decoded sign/exponent symbol selects the */
/*  fraction distribution]                                                   */
/* Both signs of one exponent e share a context, with merged counts          */
/*   n_e = cs[e] + cs[256+e],  m_e[f] = cf[e][f] + cf[256+e][f].             */
/* Candidates: the 64 exponents with the largest n_e > 0 (lower e on ties).  */
/* Excess  E_e = 128 sum_f m_e[f]^2 - n_e^2  (n_e * E_e / n_e^2 is the       */
/* chi-square distance from the flat fraction distribution).                 */
/* Eligible iff 256 E_e > n_e^2 + 726784 n_e; score = floor(E_e / n_e).      */
/* Selected: up to cmax eligible candidates with the highest score (lower e  */
/* on ties); table ids 1..k are given in ascending e.  route[s] = id of      */
/* s mod 256 when selected, else 0 (the flat table).                         */
/* qf[(id-1)*128 + f] = normalise(m_e, M_f).                                 */
/* ------------------------------------------------------------------------ */
int bso_select_tables(const uint64_t* cs, const uint64_t* cf, uint32_t M_f, uint32_t cmax,
                      uint32_t* route /*512*/, uint32_t* n_tables, uint32_t* qf /*cmax*128*/) {
    if (cmax > BSO_MAX_TABLES) return BSO_EINVAL;
    uint64_t ne[256];
    int used[256];
    for (uint32_t e = 0; e < 256; e++) { ne[e] = cs[e] + cs[256 + e]; used[e] = 0; }
    /* candidates by count */
    uint32_t cand[BSO_CANDIDATES];
    uint32_t nc = 0;
    while (nc < BSO_CANDIDATES) {
        uint32_t best = 256;
        for (uint32_t e = 0; e < 256; e++) {
            if (used[e] || ne[e] == 0) continue;
            if (best == 256 || ne[e] > ne[best]) best = e;
        }
        if (best == 256) break;
        used[best] = 1;
        cand[nc++] = best;
    }
    /* score eligible candidates */
    uint64_t score[BSO_CANDIDATES];
    int eligible[BSO_CANDIDATES];
    for (uint32_t k = 0; k < nc; k++) {
        uint32_t e = cand[k];
        unsigned __int128 n = ne[e];
        unsigned __int128 sq = 0;
        for (uint32_t f = 0; f < 128; f++) {
            unsigned __int128 m = (unsigned __int128)cf[e * 128 + f] + cf[(256 + e) * 128 + f];
            sq += m * m;
        }
        unsigned __int128 E = 128 * sq - n * n;
        eligible[k] = (256 * E > n * n + (unsigned __int128)726784 * n);
        score[k] = (uint64_t)(E / n);
    }
    /* pick the top cmax by score */
    int picked[256];
    for (uint32_t e = 0; e < 256; e++) picked[e] = 0;
    uint32_t k_sel = 0;
    int taken[BSO_CANDIDATES];
    for (uint32_t k = 0; k < nc; k++) taken[k] = 0;
    while (k_sel < cmax) {
        int best = -1;
        for (uint32_t k = 0; k < nc; k++) {
            if (!eligible[k] || taken[k]) continue;
            if (best < 0 || score[k] > score[best] ||
                (score[k] == score[best] && cand[k] < cand[best])) best = (int)k;
        }
        if (best < 0) break;
        taken[best] = 1;
        picked[cand[best]] = 1;
        k_sel++;
    }
    /* ids in ascending exponent order, tables normalised from merged counts */
    uint32_t id_of[256];
    uint32_t id = 0;
    for (uint32_t e = 0; e < 256; e++) {
        id_of[e] = 0;
        if (!picked[e]) continue;
        id++;
        id_of[e] = id;
        uint64_t m[128];
        for (uint32_t f = 0; f < 128; f++) m[f] = cf[e * 128 + f] + cf[(256 + e) * 128 + f];
        int rc = bso_normalise(m, 128, M_f, qf + (id - 1) * 128);
        if (rc) return rc;
    }
    for (uint32_t s = 0; s < 512; s++) route[s] = cs[s] ? id_of[s % 256] : 0;
    *n_tables = id;
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* floor(65536 log2 q) for 1 <= q <= 65536 (container rule, integer only).   */
/* Binary logarithm by repeated squaring: with q = 2^k r, r in [1, 2), each  */
/* squaring of r doubles its logarithm; r >= 2 after a squaring means the   */
/* next fraction bit is 1 (and r is halved).  r is held in fixed point with  */
/* 62 fraction bits; the products are exact in 128 bits and truncated back. */
/* ------------------------------------------------------------------------ */
uint32_t bso_log2_q16(uint32_t q) {
    if (q == 0) return 0;
    uint32_t k = 0;
    while ((q >> (k + 1)) != 0) k++;
    unsigned __int128 r = (unsigned __int128)q << (62 - k);   /* q / 2^k in Q62 */
    uint32_t bits = 0;
    for (int i = 0; i < 16; i++) {
        r = (r * r) >> 62;
        bits <<= 1;
        if (r >= ((unsigned __int128)2 << 62)) { bits |= 1; r >>= 1; }
    }
    return (k << 16) | bits;
}

/* ------------------------------------------------------------------------ */
/* Layout 2: choice of the coded tables for h = f >> 4 (container rule).      */
/* Both signs of an exponent e share a context, with merged counts           */
/*   n_e = cs[e] + cs[256+e],  m_e[h] = sum over f = 16h .. 16h+15 of         */
/*   cf[e][f] + cf[256+e][f].                                                 */
/* Candidate table: q_e = normalise(m_e, M_h) over the 8 values of h.        */
/* Bits it saves against the flat table (q = 2^(M_h-3) for every h), in     */
/* units of 2^-16 bit:                                                       */
/*   D_e = sum over h with m_e[h] > 0 of m_e[h] (L(q_e[h]) - 65536 (M_h-3))  */
/* with L(q) = floor(65536 log2 q).  Eligible iff D_e > 65536 * 64 (the      */
/* table's 8 bytes).  Selected: up to cmax eligible exponents with the       */
/* largest D_e (lower e on ties); ids 1..k in ascending e.  route[s] = id of */
/* s mod 256 when selected, else 0.  qh[(id-1)*8 + h] = q_e[h].              */
/* ------------------------------------------------------------------------ */
int bso_select_htables(const uint64_t* cs, const uint64_t* cf, uint32_t M_h, uint32_t cmax,
                       uint32_t* route /*512*/, uint32_t* n_tables, uint32_t* qh /*cmax*8*/) {
    if (cmax > BSO_MAX_HTABLES || M_h < 4 || M_h > 5) return BSO_EINVAL;
    __int128 saved[256];
    int eligible[256];
    uint32_t qe[256][8];
    for (uint32_t e = 0; e < 256; e++) {
        eligible[e] = 0;
        saved[e] = 0;
        uint64_t m[8];
        uint64_t n_e = cs[e] + cs[256 + e];
        for (uint32_t h = 0; h < 8; h++) {
            m[h] = 0;
            for (uint32_t f = 16 * h; f < 16 * h + 16; f++) m[h] += cf[e * 128 + f] + cf[(256 + e) * 128 + f];
        }
        if (n_e == 0) continue;
        int rc = bso_normalise(m, 8, M_h, qe[e]);
        if (rc) return rc;
        for (uint32_t h = 0; h < 8; h++) {
            if (m[h] == 0) continue;
            saved[e] += (__int128)m[h] * ((int64_t)bso_log2_q16(qe[e][h]) - 65536 * (int64_t)(M_h - 3));
        }
        eligible[e] = saved[e] > (__int128)65536 * 64;
    }
    int picked[256];
    for (uint32_t e = 0; e < 256; e++) picked[e] = 0;
    for (uint32_t k = 0; k < cmax; k++) {
        int best = -1;
        for (uint32_t e = 0; e < 256; e++) {
            if (!eligible[e] || picked[e]) continue;
            if (best < 0 || saved[e] > saved[best]) best = (int)e;
        }
        if (best < 0) break;
        picked[best] = 1;
    }
    uint32_t id_of[256];
    uint32_t id = 0;
    for (uint32_t e = 0; e < 256; e++) {
        id_of[e] = 0;
        if (!picked[e]) continue;
        id++;
        id_of[e] = id;
        for (uint32_t h = 0; h < 8; h++) qh[(id - 1) * 8 + h] = qe[e][h];
    }
    for (uint32_t s = 0; s < 512; s++) route[s] = cs[s] ? id_of[s % 256] : 0;
    *n_tables = id;
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* Lane/chunk shape of a record (container rule).                            */
/* Records of n >= Wmax weights use W = Wmax, K = Kmax.  A smaller record is */
/* one chunk whose lane count is the smallest power of two that keeps the   */
/* weights per lane at or below Wmax/Kmax (at most Kmax), with W = n rounded */
/* up to a multiple of 8K.                                                   */
/* ------------------------------------------------------------------------ */
int bso_record_shape(uint64_t n, uint32_t Wmax, uint32_t Kmax, uint32_t* W, uint32_t* K) {
    if (Kmax == 0 || Wmax == 0 || Wmax % (8 * Kmax)) return BSO_EINVAL;
    if (n >= Wmax) { *W = Wmax; *K = Kmax; return BSO_OK; }
    uint64_t per_lane = Wmax / Kmax;
    uint64_t need = (n + per_lane - 1) / per_lane;
    uint32_t k = 1;
    while (k < need && k < Kmax) k *= 2;
    if (n == 0) k = 1;
    *K = k;
    *W = (uint32_t)round_up(n ? n : 1, 8 * (uint64_t)k);
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* The rANS coder, one symbol at a time.                                     */
/* A table is (M, A, q[0..A)); cum is the running sum in symbol order.       */
/* ------------------------------------------------------------------------ */
typedef struct {
    uint32_t M;
    uint32_t A;
    const uint32_t* q;
} bso_table;

static uint32_t table_cum(const bso_table* t, uint32_t sym) {
    uint32_t c = 0;
    for (uint32_t i = 0; i < sym; i++) c += t->q[i];
    return c;
}

/* Encode one symbol into state *x; flushed 16-bit words are appended to a   */
/* growable list (in emission order, reversed later).                        */
typedef struct { uint16_t* w; uint64_t n, cap; } wordlist;

static int wl_push(wordlist* wl, uint16_t v) {
    if (wl->n == wl->cap) {
        uint64_t nc = wl->cap ? wl->cap * 2 : 1024;
        uint16_t* p = (uint16_t*)realloc(wl->w, nc * sizeof(uint16_t));
        if (!p) return BSO_ENOMEM;
        wl->w = p; wl->cap = nc;
    }
    wl->w[wl->n++] = v;
    return BSO_OK;
}

static int enc_symbol(uint32_t* x, const bso_table* t, uint32_t sym, wordlist* out) {
    uint32_t q = t->q[sym];
    if (q == 0) return BSO_EINVAL;
    uint32_t cum = table_cum(t, sym);
    uint64_t x_max = (uint64_t)q << (32 - t->M);
    if ((uint64_t)*x >= x_max) {
        int rc = wl_push(out, (uint16_t)(*x & 0xFFFFu));
        if (rc) return rc;
        *x >>= 16;
    }
    *x = (*x / q) * (1u << t->M) + (*x % q) + cum;
    return BSO_OK;
}

/* Decode one symbol from state *x, then refill from words[*pos] if needed. */
static int dec_symbol(uint32_t* x, const bso_table* t, const uint16_t* words, uint64_t nw,
                      uint64_t* pos, uint32_t* sym) {
    uint32_t slot = *x & ((1u << t->M) - 1u);
    uint32_t cum = 0, s = 0;
    while (s < t->A && !(cum <= slot && slot < cum + t->q[s])) { cum += t->q[s]; s++; }
    if (s == t->A) return BSO_ECORRUPT;
    *sym = s;
    *x = t->q[s] * (*x >> t->M) + slot - cum;
    if (*x < BSO_L) {
        if (*pos >= nw) return BSO_ECORRUPT;
        *x = (*x << 16) | words[*pos];
        *pos += 1;
    }
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* Generic interleaved coder over an explicit schedule (used by the pins):   */
/* nsteps sub-steps x K lanes; syms[step*K+l] = -1 where a lane is idle;     */
/* tab_of[step*K+l] picks the table.  Encoding walks the sub-steps from last */
/* to first and, inside one, the lanes from K-1 down to 0; the emitted words */
/* are then reversed, so decoding walks everything forwards.  Every lane     */
/* starts at init[l] (NULL: at L).                                           */
/* ------------------------------------------------------------------------ */
int bso_sched_encode(uint32_t K, uint32_t nsteps, const int32_t* syms, const uint32_t* tab_of,
                     const uint32_t* tabM, const uint32_t* tabA, const uint32_t* tabq, uint32_t ntab,
                     const uint32_t* init, uint32_t* states, uint16_t* words, uint64_t cap, uint64_t* nw) {
    bso_table* tabs = (bso_table*)malloc(sizeof(bso_table) * (ntab ? ntab : 1));
    if (!tabs) return BSO_ENOMEM;
    uint64_t off = 0;
    for (uint32_t i = 0; i < ntab; i++) { tabs[i].M = tabM[i]; tabs[i].A = tabA[i]; tabs[i].q = tabq + off; off += tabA[i]; }
    wordlist wl = {0, 0, 0};
    for (uint32_t l = 0; l < K; l++) states[l] = init ? init[l] : BSO_L;
    int rc = BSO_OK;
    for (int64_t st = (int64_t)nsteps - 1; st >= 0 && !rc; st--) {
        for (int64_t l = (int64_t)K - 1; l >= 0 && !rc; l--) {
            int32_t s = syms[(uint64_t)st * K + (uint64_t)l];
            if (s < 0) continue;
            rc = enc_symbol(&states[l], &tabs[tab_of[(uint64_t)st * K + (uint64_t)l]], (uint32_t)s, &wl);
        }
    }
    if (!rc) {
        if (wl.n > cap) rc = BSO_ENOSPACE;
        else for (uint64_t i = 0; i < wl.n; i++) words[i] = wl.w[wl.n - 1 - i];
        *nw = wl.n;
    }
    free(wl.w); free(tabs);
    return rc;
}

int bso_sched_decode(uint32_t K, uint32_t nsteps, const int32_t* active, const uint32_t* tab_of,
                     const uint32_t* tabM, const uint32_t* tabA, const uint32_t* tabq, uint32_t ntab,
                     const uint32_t* states_in, const uint16_t* words, uint64_t nw,
                     int32_t* syms_out, uint32_t* states_out) {
    bso_table* tabs = (bso_table*)malloc(sizeof(bso_table) * (ntab ? ntab : 1));
    if (!tabs) return BSO_ENOMEM;
    uint64_t off = 0;
    for (uint32_t i = 0; i < ntab; i++) { tabs[i].M = tabM[i]; tabs[i].A = tabA[i]; tabs[i].q = tabq + off; off += tabA[i]; }
    for (uint32_t l = 0; l < K; l++) states_out[l] = states_in[l];
    uint64_t pos = 0;
    int rc = BSO_OK;
    for (uint64_t st = 0; st < nsteps && !rc; st++) {
        for (uint32_t l = 0; l < K && !rc; l++) {
            uint64_t i = st * K + l;
            syms_out[i] = -1;
            if (!active[i]) continue;
            uint32_t sym;
            rc = dec_symbol(&states_out[l], &tabs[tab_of[i]], words, nw, &pos, &sym);
            if (!rc) syms_out[i] = (int32_t)sym;
        }
    }
    free(tabs);
    if (!rc && pos != nw) rc = BSO_ECORRUPT;
    return rc;
}

/* ------------------------------------------------------------------------ */
/* One chunk of a BF16 record.                                               */
/* Weight j of the chunk: group g = j / 8, position p = j mod 8, lane        */
/* l = g mod K, macro-step t = g / K.  A lane's symbols are, for t then p    */
/* ascending, the s symbol of the weight followed by its f symbol.  The      */
/* sub-step is (t, p, phase); lane l takes part iff 8(tK + l) + p < n_c.     */
/* The K lanes are split into S streams of P = K/S consecutive lanes; each   */
/* stream has its own word sequence, in which a sub-step's refills come in   */
/* ascending lane order.  The coder below handles the lanes [l0, l1) of one  */
/* stream.                                                                   */
/* Start states.  A lane's last group holds c = min(8, weights left) weights */
/* and its last m = min(4, c) weights carry only their s symbol in the      */
/* stream: their 7-bit fractions are the low 7m bits of the lane's start    */
/* state, the first of them (in decode order) lowest, under a leading one   */
/* at bit max(16, 7m).  The fractions are close to uniform, so holding them */
/* raw costs about what coding them would, while the state itself carries   */
/* some 7m bits that would otherwise cost stream words.  The decoder finds  */
/* them in its final state.  A lane without weights starts, and must end,   */
/* at L.                                                                     */
/* ------------------------------------------------------------------------ */

/* m for lane l, and through j0 the chunk index of the first of its m        */
/* weights (they are j0 .. j0 + m - 1); 0 for an empty lane.                 */
static uint32_t lane_raw_fractions(uint32_t n_c, uint32_t K, uint32_t l, uint64_t* j0) {
    uint64_t groups = ((uint64_t)n_c + 7) / 8;
    *j0 = 0;
    if (l >= groups) return 0;
    uint64_t g = l + (uint64_t)K * ((groups - 1 - l) / K);   /* the lane's last group */
    uint64_t end = 8 * g + 8 < n_c ? 8 * g + 8 : (uint64_t)n_c;
    uint64_t c = end - 8 * g;
    uint32_t m = c < 4 ? (uint32_t)c : 4u;
    *j0 = end - m;
    return m;
}

/* bit of the leading one of a start state that holds m fractions */
static uint32_t start_lead(uint32_t m) { return 7 * m > 16 ? 7 * m : 16; }

/* is chunk weight j of lane l one whose fraction is in the start state? */
static int raw_fraction(uint32_t n_c, uint32_t K, uint32_t l, uint64_t j) {
    uint64_t j0;
    uint32_t m = lane_raw_fractions(n_c, K, l, &j0);
    return m > 0 && j >= j0 && j < j0 + m;
}
typedef struct {
    uint32_t M_s, M_f;
    uint32_t qs[512];
    uint32_t route[512];
    uint32_t n_tables;
    uint32_t qf[1 + BSO_MAX_TABLES][128]; /* [0] is the flat table */
    uint32_t layout;                      /* 1, 2 or 3 */
    uint32_t qh[1 + BSO_MAX_HTABLES][8];  /* layout 2 (M_f holds M_h): [0] is the flat table */
    uint32_t qt[512 * 8];                 /* layout 3 (M_f holds M_t): q of t = 8 s + h */
} bso_model;

static int chunk_encode(const bso_model* md, const uint16_t* w, uint32_t n_c, uint32_t K,
                        uint32_t l0, uint32_t l1, uint32_t* states, wordlist* wl) {
    bso_table ts = { md->M_s, 512, md->qs };
    uint32_t groups = (n_c + 7) / 8;
    uint32_t T = (groups + K - 1) / K;
    for (uint32_t l = l0; l < l1; l++) {
        uint64_t j0;
        uint32_t m = lane_raw_fractions(n_c, K, l, &j0);
        uint32_t x = m ? 1u << start_lead(m) : BSO_L;
        for (uint32_t i = 0; i < m; i++) x |= bso_symbol_f(w[j0 + i]) << (7 * i);
        states[l] = x;
    }
    for (int64_t t = (int64_t)T - 1; t >= 0; t--) {
        for (int p = 7; p >= 0; p--) {
            for (int phase = 1; phase >= 0; phase--) {
                for (int64_t l = (int64_t)l1 - 1; l >= (int64_t)l0; l--) {
                    uint64_t j = 8 * ((uint64_t)t * K + (uint64_t)l) + (uint64_t)p;
                    if (j >= n_c || (phase == 1 && raw_fraction(n_c, K, (uint32_t)l, j))) continue;
                    uint32_t s = bso_symbol_s(w[j]);
                    int rc;
                    if (phase == 0) {
                        rc = enc_symbol(&states[l], &ts, s, wl);
                    } else {
                        bso_table tf = { md->M_f, 128, md->qf[md->route[s]] };
                        rc = enc_symbol(&states[l], &tf, bso_symbol_f(w[j]), wl);
                    }
                    if (rc) return rc;
                }
            }
        }
    }
    return BSO_OK;
}

static int chunk_decode(const bso_model* md, const uint32_t* states_in, const uint16_t* words,
                        uint64_t nw, uint32_t n_c, uint32_t K, uint32_t l0, uint32_t l1, uint16_t* out) {
    bso_table ts = { md->M_s, 512, md->qs };
    uint32_t groups = (n_c + 7) / 8;
    uint32_t T = (groups + K - 1) / K;
    uint32_t* x = (uint32_t*)malloc(sizeof(uint32_t) * K);
    uint32_t* s_now = (uint32_t*)malloc(sizeof(uint32_t) * K);
    if (!x || !s_now) { free(x); free(s_now); return BSO_ENOMEM; }
    for (uint32_t l = l0; l < l1; l++) x[l] = states_in[l];
    uint64_t pos = 0;
    int rc = BSO_OK;
    for (uint32_t t = 0; t < T && !rc; t++) {
        for (uint32_t p = 0; p < 8 && !rc; p++) {
            for (int phase = 0; phase < 2 && !rc; phase++) {
                for (uint32_t l = l0; l < l1 && !rc; l++) {
                    uint64_t j = 8 * ((uint64_t)t * K + l) + p;
                    if (j >= n_c) continue;
                    int raw = raw_fraction(n_c, K, l, j);
                    if (phase == 1 && raw) continue;
                    uint32_t sym;
                    if (phase == 0) {
                        rc = dec_symbol(&x[l], &ts, words, nw, &pos, &sym);
                        s_now[l] = sym;
                        if (!rc && raw) out[j] = bso_combine(sym, 0);   /* fraction added at the end */
                    } else {
                        bso_table tf = { md->M_f, 128, md->qf[md->route[s_now[l]]] };
                        rc = dec_symbol(&x[l], &tf, words, nw, &pos, &sym);
                        if (!rc) out[j] = bso_combine(s_now[l], sym);
                    }
                }
            }
        }
    }
    /* every lane ends at the state its encoder started from: the leading one
       over its m fractions (nothing else set), or L for an empty lane */
    for (uint32_t l = l0; l < l1 && !rc; l++) {
        uint64_t j0;
        uint32_t m = lane_raw_fractions(n_c, K, l, &j0);
        if (m == 0) { if (x[l] != BSO_L) rc = BSO_ECORRUPT; continue; }
        uint32_t lead = start_lead(m);
        if ((x[l] >> lead) != 1u || (x[l] - (1u << lead)) >= (1u << (7 * m))) { rc = BSO_ECORRUPT; continue; }
        for (uint32_t i = 0; i < m; i++) out[j0 + i] = (uint16_t)(out[j0 + i] | ((x[l] >> (7 * i)) & 0x7Fu));
    }
    if (!rc && pos != nw) rc = BSO_ECORRUPT;
    free(x); free(s_now);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Layout 2: one chunk, one renormalisation per weight.                      */
/* The lanes, groups, macro-steps, streams and word order are those of       */
/* layout 1, with one sub-step per weight: (t, p).  In a sub-step a lane     */
/* decodes s with the s-table (precision M_s) and then h = f >> 4 with the   */
/* table route[s] (precision M_h = 16 - M_s), with no renormalisation in     */
/* between; then, if its state is below L, it takes one word.  In its last  */
/* group (c = min(8, weights left) weights) a lane decodes s only: the h of  */
/* those c weights are the low 3c bits of its start state (the first weight */
/* lowest) under a leading one at bit max(16, 3c), read off the state it     */
/* ends in.  The low fraction bits l = f & 15 are not in the stream.         */
/* ------------------------------------------------------------------------ */

/* The rANS coding step of one symbol, without renormalisation. */
static void code_step(uint32_t* x, const bso_table* t, uint32_t sym) {
    uint32_t q = t->q[sym], cum = table_cum(t, sym);
    *x = (*x / q) * (1u << t->M) + (*x % q) + cum;
}

/* Its inverse: the symbol in the low M bits of *x, and the state before it. */
static int decode_step(uint32_t* x, const bso_table* t, uint32_t* sym) {
    uint32_t slot = *x & ((1u << t->M) - 1u);
    uint32_t cum = 0, s = 0;
    while (s < t->A && !(cum <= slot && slot < cum + t->q[s])) { cum += t->q[s]; s++; }
    if (s == t->A) return BSO_ECORRUPT;
    *sym = s;
    *x = t->q[s] * (*x >> t->M) + slot - cum;
    return BSO_OK;
}

/* Encode the pair (s, h): one flush check for both symbols, with the joint */
/* frequency q_s q_h at precision M_s + M_h; then h is coded, then s (the   */
/* decoder takes s first).                                                   */
static int enc_pair_words(uint32_t* x, const bso_table* ts, uint32_t s, const bso_table* th, uint32_t h,
                          wordlist* out) {
    uint64_t q = (uint64_t)ts->q[s] * th->q[h];
    if (q == 0) return BSO_EINVAL;
    uint64_t x_max = q << (32 - ts->M - th->M);
    if ((uint64_t)*x >= x_max) {
        int rc = wl_push(out, (uint16_t)(*x & 0xFFFFu));
        if (rc) return rc;
        *x >>= 16;
    }
    code_step(x, th, h);
    code_step(x, ts, s);
    return BSO_OK;
}

/* the lane's last group and the number of weights c in it (0: no weights) */
static uint32_t lane_last_group(uint32_t n_c, uint32_t K, uint32_t l, uint64_t* g_last) {
    uint64_t groups = ((uint64_t)n_c + 7) / 8;
    *g_last = 0;
    if (l >= groups) return 0;
    uint64_t g = l + (uint64_t)K * ((groups - 1 - l) / K);
    *g_last = g;
    uint64_t end = 8 * g + 8 < n_c ? 8 * g + 8 : (uint64_t)n_c;
    return (uint32_t)(end - 8 * g);
}

static uint32_t split_lead(uint32_t c) { return 3 * c > 16 ? 3 * c : 16; }

/* Layout 3: the joint table's cumulative frequencies in t order and its     */
/* slot -> symbol map (the slots of t are cum[t] .. cum[t] + q[t] - 1),      */
/* built once per chunk from qt (whose sum is 2^M_t).                        */
typedef struct {
    uint32_t cum[512 * 8];
    uint16_t sym[1u << BSO_MT];
} joint_tab;

static void joint_build(const bso_model* md, joint_tab* jt) {
    uint32_t c = 0;
    for (uint32_t t = 0; t < 512 * 8; t++) {
        jt->cum[t] = c;
        for (uint32_t k = 0; k < md->qt[t] && c + k < (1u << BSO_MT); k++) jt->sym[c + k] = (uint16_t)t;
        c += md->qt[t];
    }
}

/* Encode the joint symbol t: the flush check with its own q at M_t, then    */
/* the coding step (as enc_symbol, with the cumulative frequency looked up). */
static int enc_joint(uint32_t* x, const bso_model* md, const joint_tab* jt, uint32_t t, wordlist* out) {
    uint32_t q = md->qt[t];
    if (q == 0) return BSO_EINVAL;
    if ((uint64_t)*x >= ((uint64_t)q << (32 - BSO_MT))) {
        int rc = wl_push(out, (uint16_t)(*x & 0xFFFFu));
        if (rc) return rc;
        *x >>= 16;
    }
    *x = (*x / q) * (1u << BSO_MT) + (*x % q) + jt->cum[t];
    return BSO_OK;
}

/* Its inverse: t from the low M_t bits of *x, and the state before it. */
static void dec_joint(uint32_t* x, const bso_model* md, const joint_tab* jt, uint32_t* t) {
    uint32_t slot = *x & ((1u << BSO_MT) - 1u);
    *t = jt->sym[slot];
    *x = md->qt[*t] * (*x >> BSO_MT) + slot - jt->cum[*t];
}

static int chunk_encode_split(const bso_model* md, const uint16_t* w, uint32_t n_c, uint32_t K,
                              uint32_t l0, uint32_t l1, uint32_t* states, wordlist* wl) {
    bso_table ts = { md->M_s, 512, md->qs };
    uint32_t groups = (n_c + 7) / 8;
    uint32_t T = (groups + K - 1) / K;
    joint_tab* jt = NULL;
    if (md->layout == 3) {
        jt = (joint_tab*)malloc(sizeof(joint_tab));
        if (!jt) return BSO_ENOMEM;
        joint_build(md, jt);
    }
    for (uint32_t l = l0; l < l1; l++) {
        uint64_t g;
        uint32_t c = lane_last_group(n_c, K, l, &g);
        uint32_t x = c ? 1u << split_lead(c) : BSO_L;
        for (uint32_t i = 0; i < c; i++) x |= (bso_symbol_f(w[8 * g + i]) >> 4) << (3 * i);
        states[l] = x;
    }
    for (int64_t t = (int64_t)T - 1; t >= 0; t--) {
        for (int p = 7; p >= 0; p--) {
            for (int64_t l = (int64_t)l1 - 1; l >= (int64_t)l0; l--) {
                uint64_t j = 8 * ((uint64_t)t * K + (uint64_t)l) + (uint64_t)p;
                if (j >= n_c) continue;
                uint64_t g;
                lane_last_group(n_c, K, (uint32_t)l, &g);
                uint32_t s = bso_symbol_s(w[j]);
                int rc;
                if (j / 8 == g) {
                    rc = enc_symbol(&states[l], &ts, s, wl);
                } else if (md->layout == 3) {
                    rc = enc_joint(&states[l], md, jt, 8 * s + (bso_symbol_f(w[j]) >> 4), wl);
                } else {
                    bso_table th = { md->M_f, 8, md->qh[md->route[s]] };
                    rc = enc_pair_words(&states[l], &ts, s, &th, bso_symbol_f(w[j]) >> 4, wl);
                }
                if (rc) { free(jt); return rc; }
            }
        }
    }
    free(jt);
    return BSO_OK;
}

/* Decodes s and h of every weight of lanes [l0, l1) into out[j] = s << 7 |  */
/* h << 4 (the low fraction bits are added by the caller from the plane).    */
static int chunk_decode_split(const bso_model* md, const uint32_t* states_in, const uint16_t* words,
                              uint64_t nw, uint32_t n_c, uint32_t K, uint32_t l0, uint32_t l1, uint16_t* out) {
    bso_table ts = { md->M_s, 512, md->qs };
    uint32_t groups = (n_c + 7) / 8;
    uint32_t T = (groups + K - 1) / K;
    uint32_t* x = (uint32_t*)malloc(sizeof(uint32_t) * K);
    joint_tab* jt = md->layout == 3 ? (joint_tab*)malloc(sizeof(joint_tab)) : NULL;
    if (!x || (md->layout == 3 && !jt)) { free(x); free(jt); return BSO_ENOMEM; }
    if (jt) joint_build(md, jt);
    for (uint32_t l = l0; l < l1; l++) x[l] = states_in[l];
    uint64_t pos = 0;
    int rc = BSO_OK;
    for (uint32_t t = 0; t < T && !rc; t++) {
        for (uint32_t p = 0; p < 8 && !rc; p++) {
            for (uint32_t l = l0; l < l1 && !rc; l++) {
                uint64_t j = 8 * ((uint64_t)t * K + l) + p;
                if (j >= n_c) continue;
                uint64_t g;
                lane_last_group(n_c, K, l, &g);
                uint32_t s, h = 0;
                if (md->layout == 3 && j / 8 != g) {
                    uint32_t t;
                    dec_joint(&x[l], md, jt, &t);
                    s = t >> 3;
                    h = t & 7u;
                } else {
                    rc = decode_step(&x[l], &ts, &s);
                    if (!rc && j / 8 != g) {
                        bso_table th = { md->M_f, 8, md->qh[md->route[s]] };
                        rc = decode_step(&x[l], &th, &h);
                    }
                }
                if (rc) break;
                out[j] = (uint16_t)((s << 7) | (h << 4));
                if (x[l] < BSO_L) {
                    if (pos >= nw) { rc = BSO_ECORRUPT; break; }
                    x[l] = (x[l] << 16) | words[pos++];
                }
            }
        }
    }
    /* every lane ends at its start state: the leading one over the h of its
       last group (nothing else set), or L for a lane without weights */
    for (uint32_t l = l0; l < l1 && !rc; l++) {
        uint64_t g;
        uint32_t c = lane_last_group(n_c, K, l, &g);
        if (c == 0) { if (x[l] != BSO_L) rc = BSO_ECORRUPT; continue; }
        uint32_t lead = split_lead(c);
        if ((x[l] >> lead) != 1u || (x[l] - (1u << lead)) >= (1u << (3 * c))) { rc = BSO_ECORRUPT; continue; }
        for (uint32_t i = 0; i < c; i++) out[8 * g + i] = (uint16_t)(out[8 * g + i] | (((x[l] >> (3 * i)) & 7u) << 4));
    }
    if (!rc && pos != nw) rc = BSO_ECORRUPT;
    free(x);
    free(jt);
    return rc;
}

/* The chunk's plane of low fraction bits: one 32-bit word per group of 8    */
/* weights, group g at byte 4g; the low bits of position p of the group at  */
/* bit 16 (p mod 2) + 4 (p div 2) (even positions in the low half, odd ones */
/* in the high half); positions past the chunk's end hold 0.                */
static uint32_t low_bit_pos(uint32_t p) { return 16 * (p % 2) + 4 * (p / 2); }

/* bytes of a chunk's plane of low fraction bits, padded to 16 */
static uint64_t plane_bytes(uint32_t n_c) { return round_up(4 * (((uint64_t)n_c + 7) / 8), 16); }

/* ------------------------------------------------------------------------ */
/* Byte buffer for the container                                             */
/* ------------------------------------------------------------------------ */
typedef struct { uint8_t* p; uint64_t n, cap; } bytebuf;

static int bb_reserve(bytebuf* b, uint64_t need) {
    if (need <= b->cap) return BSO_OK;
    uint64_t nc = b->cap ? b->cap : 4096;
    while (nc < need) nc *= 2;
    uint8_t* p = (uint8_t*)realloc(b->p, nc);
    if (!p) return BSO_ENOMEM;
    memset(p + b->cap, 0, nc - b->cap);
    b->p = p; b->cap = nc;
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* Final lane states of a chunk, packed.  A state x in [2^16, 2^32) is       */
/* written as its length code e = floor(log2 x) - 16 (0..15, one nibble per */
/* lane, lane l in the low nibble of byte l/2 when l is even) and its 16 + e */
/* bits below the leading one.  Those bits are concatenated in lane order,   */
/* least significant first, from bit 0 of the mantissa block.                */
/* ------------------------------------------------------------------------ */
static uint32_t state_code(uint32_t x) {
    uint32_t e = 0;
    while (e < 15 && (x >> (17 + e)) != 0) e++;
    return e;
}

/* bytes of the nibble block of K lanes; 16-bit units of the state bits of P
   lanes whose codes sum to esum */
static uint64_t code_block_bytes(uint32_t K) { return round_up(((uint64_t)K + 1) / 2, 16); }
static uint64_t mant_units(uint32_t P, uint64_t esum) { return (16ull * P + esum + 15) / 16; }

static void put_bits(uint8_t* b, uint64_t off, uint32_t v, uint32_t len) {
    for (uint32_t i = 0; i < len; i++) {
        uint64_t bit = off + i;
        if ((v >> i) & 1u) b[bit / 8] |= (uint8_t)(1u << (bit % 8));
    }
}

static uint32_t get_bits(const uint8_t* b, uint64_t off, uint32_t len) {
    uint32_t v = 0;
    for (uint32_t i = 0; i < len; i++) {
        uint64_t bit = off + i;
        v |= (uint32_t)((b[bit / 8] >> (bit % 8)) & 1u) << i;
    }
    return v;
}

/* ------------------------------------------------------------------------ */
/* Layout 2: shared routing (container rule, integer only).                  */
/* [NVLC card, codec paragraph: the fraction distribution is routed from the */
/*  decoded symbol; the route byte may name any of the record's tables]      */
/* After the coded tables are chosen, each occupied exponent e that did not  */
/* get a table of its own (route 0) is routed to the table t -- the flat     */
/* table 0 or a coded table 1..n_tables -- that codes its merged h counts    */
/* m_e[h] in the fewest bits, counted in units of 2^-16 bit:                 */
/*   cost_t(e) = sum over h with m_e[h] > 0 of m_e[h] (65536 M_h - L(q_t[h])) */
/* with L(q) = floor(65536 log2 q).  A table with q_t[h] = 0 for an h that  */
/* e uses cannot code e.  The lowest cost wins, the lower id on ties (so    */
/* the flat table keeps e unless a coded table is strictly cheaper).  Both  */
/* signs of e follow: route[s] for the occupied s of exponent e.             */
/* qh holds the coded tables only: qh[(t-1)*8 + h] for t = 1..n_tables.     */
/* ------------------------------------------------------------------------ */
int bso_share_hroutes(const uint64_t* cs, const uint64_t* cf, uint32_t M_h, uint32_t n_tables, const uint32_t* qh,
                      uint32_t* route /*512*/) {
    if (M_h < 4 || M_h > 5 || n_tables > BSO_MAX_HTABLES) return BSO_EINVAL;
    for (uint32_t e = 0; e < 256; e++) {
        if (cs[e] + cs[256 + e] == 0) continue;
        if ((cs[e] && route[e]) || (cs[256 + e] && route[256 + e])) continue;   /* has its own table */
        uint64_t m[8];
        for (uint32_t h = 0; h < 8; h++) {
            m[h] = 0;
            for (uint32_t f = 16 * h; f < 16 * h + 16; f++) m[h] += cf[e * 128 + f] + cf[(256 + e) * 128 + f];
        }
        uint32_t best = 0;
        unsigned __int128 best_cost = 0;
        for (uint32_t t = 0; t <= n_tables; t++) {
            unsigned __int128 cost = 0;
            int usable = 1;
            for (uint32_t h = 0; h < 8; h++) {
                if (m[h] == 0) continue;
                uint32_t q = t == 0 ? (1u << (M_h - 3)) : qh[(t - 1) * 8 + h];
                if (q == 0) { usable = 0; break; }
                cost += (unsigned __int128)m[h] * (65536u * M_h - bso_log2_q16(q));
            }
            if (!usable) continue;
            if (t == 0 || cost < best_cost) { best = t; best_cost = cost; }
        }
        if (cs[e]) route[e] = best;
        if (cs[256 + e]) route[256 + e] = best;
    }
    return BSO_OK;
}

/* ------------------------------------------------------------------------ */
/* Encode one BF16 record body.                                              */
/* ------------------------------------------------------------------------ */
static int encode_bf16_body(const uint16_t* w, uint64_t n, uint32_t Wmax, uint32_t Kmax, uint32_t Pmax,
                            uint32_t M_s, uint32_t M_f, uint32_t cmax, uint32_t layout, bytebuf* body) {
    uint32_t W, K;
    int rc = bso_record_shape(n, Wmax, Kmax, &W, &K);
    if (rc) return rc;
    /* streams per chunk: the record's lanes in groups of at most Pmax */
    uint32_t P = K < Pmax ? K : Pmax;
    uint32_t S = K / P, log2S = 0;
    while ((1u << log2S) < S) log2S++;
    bso_model* md = (bso_model*)calloc(1, sizeof(bso_model));
    uint64_t* cs = (uint64_t*)calloc(512, sizeof(uint64_t));
    uint64_t* cf = (uint64_t*)calloc(512 * 128, sizeof(uint64_t));
    if (!md || !cs || !cf) { free(md); free(cs); free(cf); return BSO_ENOMEM; }
    md->M_s = M_s; md->M_f = M_f; md->layout = layout;
    uint32_t n_sym = 0;
    uint64_t n_chunks = n ? (n + W - 1) / W : 0;
    if (n) {
        bso_histogram(w, n, cs, cf);
        rc = bso_normalise(cs, 512, M_s, md->qs);
        if (!rc && layout == 1) rc = bso_select_tables(cs, cf, M_f, cmax, md->route, &md->n_tables, &md->qf[1][0]);
        if (!rc && layout == 2) rc = bso_select_htables(cs, cf, M_f, cmax, md->route, &md->n_tables, &md->qh[1][0]);
        if (!rc && layout == 2) rc = bso_share_hroutes(cs, cf, M_f, md->n_tables, &md->qh[1][0], md->route);
        if (!rc && layout == 3) {
            /* the joint counts of t = 8 s + h: the fraction counts of s summed
               over the low four bits */
            uint64_t* ct = (uint64_t*)calloc(512 * 8, sizeof(uint64_t));
            if (!ct) rc = BSO_ENOMEM;
            for (uint32_t t = 0; !rc && t < 512 * 8; t++)
                for (uint32_t lo = 0; lo < 16; lo++) ct[t] += cf[(t >> 3) * 128 + 16 * (t & 7u) + lo];
            if (!rc) rc = bso_normalise(ct, 512 * 8, BSO_MT, md->qt);
            free(ct);
        }
        for (uint32_t s = 0; s < 512; s++) if (cs[s]) n_sym++;
    }
    if (layout == 1) for (uint32_t f = 0; f < 128; f++) md->qf[0][f] = 1u << (M_f - 7);
    if (layout == 2) for (uint32_t h = 0; h < 8; h++) md->qh[0][h] = 1u << (M_f - 3);
    if (rc) goto done;

    /* fixed part, tables, chunk index and (S > 1) stream table */
    uint64_t off = 24;
    uint64_t tables_end = off + 4ull * n_sym;
    tables_end = round_up(tables_end + n_sym, 4);
    tables_end += layout == 3 ? 16ull * n_sym : (layout == 1 ? 256ull : 8ull) * md->n_tables;
    uint64_t index_off = round_up(tables_end, 16);
    uint64_t stab_off = index_off + 16 * n_chunks;
    uint64_t payload_off = round_up(stab_off + 4ull * (S - 1) * n_chunks, 16);
    rc = bb_reserve(body, payload_off);
    if (rc) goto done;
    body->n = payload_off;
    uint8_t* b = body->p;
    put32(b + 0, W); put32(b + 4, K); put32(b + 8, (uint32_t)n_chunks);
    b[12] = (uint8_t)M_s; b[13] = (uint8_t)M_f; b[14] = (uint8_t)md->n_tables; b[15] = (uint8_t)log2S;
    put32(b + 16, n_sym); put32(b + 20, layout == 1 ? 0 : layout);
    uint64_t k = 0;
    for (uint32_t s = 0; s < 512; s++) {
        if (!cs[s]) continue;
        put16(b + off + 4 * k, s);
        put16(b + off + 4 * k + 2, md->qs[s]);
        b[off + 4ull * n_sym + k] = (uint8_t)md->route[s];
        k++;
    }
    uint64_t ft = round_up(off + 4ull * n_sym + n_sym, 4);
    for (uint32_t t = 1; t <= md->n_tables; t++) {
        if (layout == 1) for (uint32_t f = 0; f < 128; f++) put16(b + ft + 256ull * (t - 1) + 2 * f, md->qf[t][f]);
        else for (uint32_t h = 0; h < 8; h++) b[ft + 8ull * (t - 1) + h] = (uint8_t)md->qh[t][h];
    }
    /* layout 3: the joint table, eight 16-bit q (h = 0..7) per occupied s in
       the order of the s list */
    if (layout == 3) {
        uint64_t kk = 0;
        for (uint32_t sy = 0; sy < 512; sy++) {
            if (!cs[sy]) continue;
            for (uint32_t h = 0; h < 8; h++) put16(b + ft + 16 * kk + 2 * h, md->qt[8 * sy + h]);
            kk++;
        }
    }

    /* chunks: the K lanes' length codes, padded to 16 bytes, then the
       streams back to back, each the state bits of its P lanes (padded to a
       16-bit unit) followed by its words; the payload is padded to 16 bytes.
       The index gives the payload's offset and the units of its stream area;
       the stream table the start unit of streams 1 .. S-1 */
    uint32_t* states = (uint32_t*)malloc(sizeof(uint32_t) * K);
    wordlist* wls = (wordlist*)calloc(S, sizeof(wordlist));
    uint64_t* units = (uint64_t*)calloc(S, sizeof(uint64_t));
    uint64_t* mu = (uint64_t*)calloc(S, sizeof(uint64_t));
    if (!states || !wls || !units || !mu) { free(states); free(wls); free(units); free(mu); rc = BSO_ENOMEM; goto done; }
    for (uint64_t c = 0; c < n_chunks && !rc; c++) {
        uint32_t n_c = (uint32_t)((n - c * W) < W ? (n - c * W) : W);
        for (uint32_t st = 0; st < S; st++) wls[st].n = 0;
        for (uint32_t st = 0; st < S && !rc; st++) {
            if (layout == 1) rc = chunk_encode(md, w + c * W, n_c, K, st * P, (st + 1) * P, states, &wls[st]);
            else rc = chunk_encode_split(md, w + c * W, n_c, K, st * P, (st + 1) * P, states, &wls[st]);
        }
        if (rc) break;
        uint64_t total = 0;
        for (uint32_t st = 0; st < S; st++) {
            uint64_t esum = 0;
            for (uint32_t l = st * P; l < (st + 1) * P; l++) esum += state_code(states[l]);
            mu[st] = mant_units(P, esum);
            units[st] = mu[st] + wls[st].n;
            total += units[st];
        }
        uint64_t start = body->n;
        /* layout 2: the plane of low fraction bits sits between the length
           codes and the stream area */
        uint64_t code_bytes = code_block_bytes(K) + (layout >= 2 ? plane_bytes(n_c) : 0);
        uint64_t end = start + round_up(code_bytes + 2 * total, 16);
        rc = bb_reserve(body, end);
        if (rc) break;
        b = body->p;
        memset(b + start, 0, end - start);
        put64(b + index_off + 16 * c, start);
        put32(b + index_off + 16 * c + 8, (uint32_t)total);
        put32(b + index_off + 16 * c + 12, 0);
        for (uint32_t l = 0; l < K; l++) b[start + l / 2] |= (uint8_t)(state_code(states[l]) << (4 * (l % 2)));
        if (layout >= 2) {
            uint8_t* plane = b + start + code_block_bytes(K);
            for (uint32_t j = 0; j < n_c; j++) {
                uint32_t g = j / 8, p = j % 8;
                uint32_t v = get32(plane + 4 * g) | ((bso_symbol_f(w[c * W + j]) & 15u) << low_bit_pos(p));
                put32(plane + 4 * g, v);
            }
        }
        uint64_t at = 0;   /* units from the start of the stream area */
        for (uint32_t st = 0; st < S; st++) {
            if (st > 0) put32(b + stab_off + 4 * ((S - 1) * c + st - 1), (uint32_t)at);
            uint8_t* area = b + start + code_bytes + 2 * at;
            uint64_t moff = 0;
            for (uint32_t l = st * P; l < (st + 1) * P; l++) {
                uint32_t e = state_code(states[l]);
                put_bits(area, moff, states[l] - (1u << (16 + e)), 16 + e);
                moff += 16 + e;
            }
            /* the encoder pushes words in reverse order of their use */
            for (uint64_t i = 0; i < wls[st].n; i++) put16(area + 2 * (mu[st] + i), wls[st].w[wls[st].n - 1 - i]);
            at += units[st];
        }
        body->n = end;
    }
    free(units); free(mu);
    for (uint32_t st = 0; st < S; st++) free(wls[st].w);
    free(wls);
    free(states);
done:
    free(md); free(cs); free(cf);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Whole container.                                                          */
/* kinds[i]: 1 = BF16 (n[i] weights at data[i]), 2 = RAW (n[i] bytes).       */
/* sha[i*32..]: sha256 of the tensor's bytes, computed by the caller.        */
/* A BF16 tensor with more than 256 occupied (sign,exp) symbols is stored    */
/* as a RAW record of its 2n bytes.                                          */
/* On success *out points to malloc'ed bytes (free with bso_free).          */
/* ------------------------------------------------------------------------ */
/* layout 1 writes a version-1 container, layout 2 a version-2 container,   */
/* layout 3 a version-3 one (every BF16 record in that layout).  Layout 2:   */
/* M_s is 11 or 12 and M_f holds M_h = 16 - M_s; cmax <= 31.  Layout 3: M_s  */
/* is 11 or 12 and M_f holds M_t = 13; cmax is not used.                     */
int bso_encode_container2(uint32_t n_tensors, const uint32_t* kinds, const void* const* data,
                          const uint64_t* n, const uint8_t* sha,
                          uint32_t Wmax, uint32_t Kmax, uint32_t Pmax, uint32_t M_s, uint32_t M_f, uint32_t cmax,
                          uint32_t layout, uint8_t** out, uint64_t* out_len) {
    if (layout == 1 && (M_s < 9 || M_s > 12 || M_f < 8 || M_f > 10 || cmax > BSO_MAX_TABLES)) return BSO_EINVAL;
    if (layout == 2 && (M_s < 11 || M_s > 12 || M_f != 16 - M_s || cmax > BSO_MAX_HTABLES)) return BSO_EINVAL;
    if (layout == 3 && (M_s < 11 || M_s > 12 || M_f != BSO_MT)) return BSO_EINVAL;
    if (layout < 1 || layout > 3) return BSO_EINVAL;
    if (!(Kmax <= 64 || Kmax == 128 || Kmax == 256 || Kmax == 512 || Kmax == 1024 || Kmax == 2048) || Kmax == 0) return BSO_EINVAL;
    if ((Kmax & (Kmax - 1)) != 0) return BSO_EINVAL;
    if (Pmax == 0 || (Pmax & (Pmax - 1)) != 0 || Pmax > Kmax || Pmax > 512) return BSO_EINVAL;
    bytebuf c = {0, 0, 0};
    uint64_t dir = BSO_HDR_BYTES;
    uint64_t pos = round_up(dir + (uint64_t)BSO_DIR_BYTES * n_tensors, 16);
    int rc = bb_reserve(&c, pos);
    if (rc) return rc;
    c.n = pos;
    uint64_t out_pos = 0;
    for (uint32_t i = 0; i < n_tensors && !rc; i++) {
        uint32_t kind = kinds[i];
        uint64_t bytes = kind == BSO_KIND_BF16 ? 2 * n[i] : n[i];
        uint64_t count = n[i];
        bytebuf body = {0, 0, 0};
        if (kind == BSO_KIND_BF16) {
            /* count occupied symbols first: too many -> verbatim */
            const uint16_t* w = (const uint16_t*)data[i];
            int seen[512];
            uint32_t occ = 0;
            for (int s = 0; s < 512; s++) seen[s] = 0;
            for (uint64_t j = 0; j < n[i]; j++) {
                uint32_t s = bso_symbol_s(w[j]);
                if (!seen[s]) { seen[s] = 1; occ++; }
            }
            if (occ > BSO_MAX_SYMS) { kind = BSO_KIND_RAW; count = bytes; }
        }
        if (kind == BSO_KIND_BF16) {
            rc = encode_bf16_body((const uint16_t*)data[i], n[i], Wmax, Kmax, Pmax, M_s, M_f, cmax, layout, &body);
        } else if (kind == BSO_KIND_RAW) {
            rc = bb_reserve(&body, bytes ? bytes : 1);
            if (!rc) { if (bytes) memcpy(body.p, data[i], bytes); body.n = bytes; }
        } else {
            rc = BSO_EINVAL;
        }
        if (rc) { free(body.p); break; }
        uint64_t rec_off = round_up(c.n, 16);
        rc = bb_reserve(&c, rec_off + body.n);
        if (rc) { free(body.p); break; }
        if (body.n) memcpy(c.p + rec_off, body.p, body.n);
        c.n = rec_off + body.n;
        free(body.p);
        uint8_t* d = c.p + dir + (uint64_t)BSO_DIR_BYTES * i;
        put32(d + 0, kind); put32(d + 4, 0);
        put64(d + 8, count);
        put64(d + 16, out_pos);
        put64(d + 24, rec_off);
        put64(d + 32, c.n - rec_off);
        memcpy(d + 40, sha + 32ull * i, 32);
        out_pos = round_up(out_pos + bytes, BSO_OUT_ALIGN);
    }
    if (rc) { free(c.p); return rc; }
    uint64_t total = round_up(c.n, 16);
    rc = bb_reserve(&c, total);
    if (rc) { free(c.p); return rc; }
    c.n = total;
    /* the decoded extent ends with the last record's bytes (no trailing pad) */
    uint64_t out_len_bytes = 0;
    for (uint32_t i = 0; i < n_tensors; i++) {
        const uint8_t* d = c.p + dir + (uint64_t)BSO_DIR_BYTES * i;
        uint64_t kind = get32(d), cnt = get64(d + 8), oo = get64(d + 16);
        uint64_t e = oo + (kind == BSO_KIND_BF16 ? 2 * cnt : cnt);
        if (e > out_len_bytes) out_len_bytes = e;
    }
    memcpy(c.p, BSO_MAGIC, 8);
    put32(c.p + 8, layout == 1 ? BSO_VERSION : layout == 2 ? BSO_VERSION2 : BSO_VERSION3);
    put32(c.p + 12, n_tensors);
    put64(c.p + 16, dir);
    put64(c.p + 24, total);
    put64(c.p + 32, out_len_bytes);
    *out = c.p;
    *out_len = total;
    return BSO_OK;
}

int bso_encode_container(uint32_t n_tensors, const uint32_t* kinds, const void* const* data,
                         const uint64_t* n, const uint8_t* sha,
                         uint32_t Wmax, uint32_t Kmax, uint32_t Pmax, uint32_t M_s, uint32_t M_f, uint32_t cmax,
                         uint8_t** out, uint64_t* out_len) {
    return bso_encode_container2(n_tensors, kinds, data, n, sha, Wmax, Kmax, Pmax, M_s, M_f, cmax, 1, out, out_len);
}

void bso_free(void* p) { free(p); }

/* ------------------------------------------------------------------------ */
/* Decode a container into out (out_cap bytes, zero-filled gaps untouched).  */
/* rec_status[i] (may be NULL) receives 0 or the error of record i.          */
/* Returns the first error, or 0.                                            */
/* ------------------------------------------------------------------------ */
static int parse_model(const uint8_t* b, uint64_t len, uint64_t n, uint32_t version, bso_model* md,
                       uint32_t* W, uint32_t* K, uint32_t* S, uint64_t* n_chunks, uint64_t* index_off) {
    if (len < 24) return BSO_EFORMAT;
    *W = get32(b); *K = get32(b + 4);
    *n_chunks = get32(b + 8);
    md->M_s = b[12]; md->M_f = b[13]; md->n_tables = b[14];
    if (b[15] > 9) return BSO_EFORMAT;
    *S = 1u << b[15];
    uint32_t n_sym = get32(b + 16);
    /* version 1: the word at +20 is 0 (layout 1); versions 2 and 3 name the
       layout there (1 or 2; version 3 also 3) */
    uint32_t lw = get32(b + 20);
    if (version == BSO_VERSION) { if (lw != 0) return BSO_EFORMAT; md->layout = 1; }
    else { if (lw < 1 || lw > (version == BSO_VERSION3 ? 3u : 2u)) return BSO_EFORMAT; md->layout = lw; }
    if (md->layout == 1 && (md->M_s < 9 || md->M_s > 12 || md->M_f < 8 || md->M_f > 10 || md->n_tables > BSO_MAX_TABLES))
        return BSO_EFORMAT;
    if (md->layout == 2 && (md->M_s < 11 || md->M_s > 12 || md->M_f != 16 - md->M_s || md->n_tables > BSO_MAX_HTABLES))
        return BSO_EFORMAT;
    if (md->layout == 3 && (md->M_s < 11 || md->M_s > 12 || md->M_f != BSO_MT || md->n_tables != 0)) return BSO_EFORMAT;
    if (*K == 0 || *W == 0 || *W % (8 * *K)) return BSO_EFORMAT;
    if (!(*K <= 64 || *K == 128 || *K == 256 || *K == 512 || *K == 1024 || *K == 2048)) return BSO_EFORMAT;
    if (*K % *S || *K / *S > 512) return BSO_EFORMAT;
    if (*n_chunks != (n + *W - 1) / *W) return BSO_EFORMAT;
    if (n_sym > BSO_MAX_SYMS || (n_sym == 0) != (n == 0)) return BSO_EFORMAT;
    uint64_t off = 24;
    uint64_t ft = round_up(off + 4ull * n_sym + n_sym, 4);
    uint64_t tab_end = ft + (md->layout == 3 ? 16ull * n_sym : (md->layout == 1 ? 256ull : 8ull) * md->n_tables);
    *index_off = round_up(tab_end, 16);
    if (*index_off + 16 * *n_chunks + 4ull * (*S - 1) * *n_chunks > len) return BSO_EFORMAT;
    memset(md->qs, 0, sizeof(md->qs));
    memset(md->route, 0, sizeof(md->route));
    uint64_t sum = 0;
    int last = -1;
    for (uint32_t k = 0; k < n_sym; k++) {
        uint32_t s = get16(b + off + 4ull * k), q = get16(b + off + 4ull * k + 2);
        if ((int)s <= last || s >= 512 || q == 0) return BSO_EFORMAT;
        last = (int)s;
        md->qs[s] = q;
        md->route[s] = b[off + 4ull * n_sym + k];
        if (md->route[s] > md->n_tables) return BSO_EFORMAT;
        sum += q;
    }
    if (n_sym && sum != (1ull << md->M_s)) return BSO_EFORMAT;
    if (md->layout == 3) {
        /* eight joint frequencies per listed s, summing to 2^M_t over all */
        memset(md->qt, 0, sizeof(md->qt));
        uint64_t tsum = 0;
        for (uint32_t k = 0; k < n_sym; k++) {
            uint32_t sy = get16(b + off + 4ull * k);
            for (uint32_t h = 0; h < 8; h++) { md->qt[8 * sy + h] = get16(b + ft + 16ull * k + 2 * h); tsum += md->qt[8 * sy + h]; }
        }
        if (n_sym && tsum != (1ull << BSO_MT)) return BSO_EFORMAT;
        return BSO_OK;
    }
    if (md->layout == 2) {
        for (uint32_t h = 0; h < 8; h++) md->qh[0][h] = 1u << (md->M_f - 3);
        for (uint32_t t = 1; t <= md->n_tables; t++) {
            uint64_t tsum = 0;
            for (uint32_t h = 0; h < 8; h++) { md->qh[t][h] = b[ft + 8ull * (t - 1) + h]; tsum += md->qh[t][h]; }
            if (tsum != (1ull << md->M_f)) return BSO_EFORMAT;
        }
        return BSO_OK;
    }
    for (uint32_t f = 0; f < 128; f++) md->qf[0][f] = 1u << (md->M_f - 7);
    for (uint32_t t = 1; t <= md->n_tables; t++) {
        uint64_t tsum = 0;
        for (uint32_t f = 0; f < 128; f++) { md->qf[t][f] = get16(b + ft + 256ull * (t - 1) + 2 * f); tsum += md->qf[t][f]; }
        if (tsum != (1ull << md->M_f)) return BSO_EFORMAT;
    }
    return BSO_OK;
}

/* Decode chunk ch of a parsed BF16 record body b (rl bytes) into out[0..n_c). */
static int decode_one_chunk(const bso_model* md, const uint8_t* b, uint64_t rl, uint64_t io, uint32_t K,
                            uint32_t S, uint64_t n_chunks, uint64_t ch, uint32_t n_c, uint16_t* out) {
    const uint8_t* e = b + io + 16 * ch;
    uint64_t po = get64(e), total = get32(e + 8);
    /* layouts 2 and 3: the plane of low fraction bits follows the length codes */
    uint64_t code_bytes = code_block_bytes(K) + (md->layout >= 2 ? plane_bytes(n_c) : 0);
    if (po % 16 || po > rl || code_bytes > rl - po || 2 * total > rl - po - code_bytes) return BSO_EFORMAT;
    const uint8_t* stab = b + io + 16 * n_chunks + 4 * (S - 1) * ch;
    uint32_t P = K / S;
    uint32_t* st = (uint32_t*)malloc(sizeof(uint32_t) * K);
    if (!st) return BSO_ENOMEM;
    int rc = BSO_OK;
    for (uint32_t s = 0; s < S && !rc; s++) {
        uint64_t from = s ? get32(stab + 4 * (s - 1)) : 0;
        uint64_t to = s + 1 < S ? get32(stab + 4 * s) : total;
        if (from > to || to > total) { rc = BSO_EFORMAT; break; }
        const uint8_t* area = b + po + code_bytes + 2 * from;
        /* the stream's lanes' states: length codes from the chunk's nibble
           block, bits from the head of the stream's area */
        uint64_t moff = 0, esum = 0;
        for (uint32_t l = s * P; l < (s + 1) * P; l++) {
            uint32_t el = (b[po + l / 2] >> (4 * (l % 2))) & 15u;
            esum += el;
        }
        uint64_t mu = mant_units(P, esum);
        if (mu > to - from) { rc = BSO_EFORMAT; break; }
        for (uint32_t l = s * P; l < (s + 1) * P; l++) {
            uint32_t el = (b[po + l / 2] >> (4 * (l % 2))) & 15u;
            st[l] = (1u << (16 + el)) | get_bits(area, moff, 16 + el);
            moff += 16 + el;
        }
        uint64_t nws = to - from - mu;
        uint16_t* words = (uint16_t*)malloc(sizeof(uint16_t) * (nws ? nws : 1));
        if (!words) { rc = BSO_ENOMEM; break; }
        for (uint64_t j = 0; j < nws; j++) words[j] = (uint16_t)get16(area + 2 * (mu + j));
        if (md->layout == 1) rc = chunk_decode(md, st, words, nws, n_c, K, s * P, (s + 1) * P, out);
        else rc = chunk_decode_split(md, st, words, nws, n_c, K, s * P, (s + 1) * P, out);
        free(words);
    }
    free(st);
    if (!rc && md->layout >= 2) {
        const uint8_t* plane = b + po + code_block_bytes(K);
        for (uint32_t j = 0; j < n_c; j++)
            out[j] = (uint16_t)(out[j] | ((get32(plane + 4 * (j / 8)) >> low_bit_pos(j % 8)) & 15u));
    }
    return rc;
}

int bso_decode_container(const uint8_t* c, uint64_t len, uint8_t* out, uint64_t out_cap, int32_t* rec_status) {
    if (len < BSO_HDR_BYTES || memcmp(c, BSO_MAGIC, 8) != 0) return BSO_EFORMAT;
    uint32_t version = get32(c + 8);
    if (version != BSO_VERSION && version != BSO_VERSION2 && version != BSO_VERSION3) return BSO_EVERSION;
    uint32_t n_rec = get32(c + 12);
    uint64_t dir = get64(c + 16);
    if (get64(c + 24) != len) return BSO_EFORMAT;
    if (dir + (uint64_t)BSO_DIR_BYTES * n_rec > len) return BSO_EFORMAT;
    if (get64(c + 32) > out_cap) return BSO_ENOSPACE;
    int first_err = BSO_OK;
    for (uint32_t i = 0; i < n_rec; i++) {
        const uint8_t* d = c + dir + (uint64_t)BSO_DIR_BYTES * i;
        uint32_t kind = get32(d);
        uint64_t n = get64(d + 8), oo = get64(d + 16), ro = get64(d + 24), rl = get64(d + 32);
        int rc = BSO_OK;
        if (ro + rl > len || ro + rl < ro) rc = BSO_EFORMAT;
        else if (kind == BSO_KIND_RAW) {
            if (oo + n > out_cap || rl < n) rc = BSO_EFORMAT;
            else if (n) memcpy(out + oo, c + ro, n);
        } else if (kind == BSO_KIND_BF16) {
            bso_model* md = (bso_model*)calloc(1, sizeof(bso_model));
            uint32_t W, K, S; uint64_t nch, io;
            if (!md) rc = BSO_ENOMEM;
            if (!rc) rc = parse_model(c + ro, rl, n, version, md, &W, &K, &S, &nch, &io);
            if (!rc && (oo + 2 * n > out_cap || oo % 16)) rc = BSO_EFORMAT;
            uint16_t* tmp = NULL;
            if (!rc && n) { tmp = (uint16_t*)malloc(sizeof(uint16_t) * W); if (!tmp) rc = BSO_ENOMEM; }
            for (uint64_t ch = 0; ch < nch && !rc; ch++) {
                uint32_t n_c = (uint32_t)((n - ch * W) < W ? (n - ch * W) : W);
                rc = decode_one_chunk(md, c + ro, rl, io, K, S, nch, ch, n_c, tmp);
                if (!rc) for (uint32_t j = 0; j < n_c; j++) put16(out + oo + 2 * (ch * W + j), tmp[j]);
            }
            free(tmp); free(md);
        } else {
            rc = BSO_EFORMAT;
        }
        if (rec_status) rec_status[i] = rc;
        if (rc && !first_err) first_err = rc;
    }
    return first_err;
}

/* ------------------------------------------------------------------------ */
/* Decode one chunk of one BF16 record (for sampled checks on big inputs).   */
/* out receives the chunk's n_c words; *n_c_out their count.                 */
/* ------------------------------------------------------------------------ */
int bso_decode_chunk(const uint8_t* c, uint64_t len, uint32_t record, uint64_t chunk,
                     uint16_t* out, uint64_t out_cap, uint64_t* n_c_out) {
    if (len < BSO_HDR_BYTES || memcmp(c, BSO_MAGIC, 8) != 0) return BSO_EFORMAT;
    uint32_t version = get32(c + 8);
    if (version != BSO_VERSION && version != BSO_VERSION2 && version != BSO_VERSION3) return BSO_EVERSION;
    uint32_t n_rec = get32(c + 12);
    uint64_t dir = get64(c + 16);
    if (record >= n_rec || dir + (uint64_t)BSO_DIR_BYTES * n_rec > len) return BSO_EINVAL;
    const uint8_t* d = c + dir + (uint64_t)BSO_DIR_BYTES * record;
    if (get32(d) != BSO_KIND_BF16) return BSO_EINVAL;
    uint64_t n = get64(d + 8), ro = get64(d + 24), rl = get64(d + 32);
    if (ro > len || rl > len - ro) return BSO_EFORMAT;
    bso_model* md = (bso_model*)calloc(1, sizeof(bso_model));
    if (!md) return BSO_ENOMEM;
    uint32_t W, K, S; uint64_t nch, io;
    int rc = parse_model(c + ro, rl, n, version, md, &W, &K, &S, &nch, &io);
    if (!rc && chunk >= nch) rc = BSO_EINVAL;
    uint64_t n_c = 0;
    if (!rc) {
        n_c = (n - chunk * W) < W ? (n - chunk * W) : W;
        if (n_c > out_cap) rc = BSO_ENOSPACE;
    }
    if (!rc) rc = decode_one_chunk(md, c + ro, rl, io, K, S, nch, chunk, (uint32_t)n_c, out);
    free(md);
    *n_c_out = n_c;
    return rc;
}

/* ======================================================================== */
/* Fixed-width lane streams (test infrastructure, like everything here).    */
/*                                                                          */
/* [NVLC card, runtime paragraphs: the measured GPU runtime derives          */
/*  fixed-width, lane-oriented streams from the canonical model once at     */
/*  initialisation, with the fraction kept as a fixed 7-bit field; the      */
/*  pages give the names and the resident size (about 71% of BF16) but not  */
/*  the layout, which is this repository's own definition.]                 */
/*                                                                          */
/* One tensor of n BF16 words.  Every weight is an 11-bit code word: a      */
/* 4-bit symbol code and its exact 7-bit fraction.  Codes 0..14 stand for   */
/* the 15 most frequent (sign, exponent) symbols of the tensor (count       */
/* descending, ties to the lower symbol); code 15 is an escape, whose       */
/* symbol is the next entry of the tensor's escape list.                    */
/*   header 96 B: "BF16FIX1", u32 version 1, u32 0, u64 n, u64 n_blocks,     */
/*     u64 escape list offset, u64 escapes, 16 B zero, 16 x u16 the symbol  */
/*     of codes 0..15 (unused entries and entry 15: 0)                      */
/*   blocks of 2048 weights, 2816 B each: lane l (0..63) holds weights      */
/*     32 l .. 32 l + 31 of the block (past n: code 0, fraction 0);         */
/*     code plane: dword k (0..3) of lane l at 4 (64 k + l), weight 8 k + i  */
/*       of the lane in bits 4 i .. 4 i + 3;                                */
/*     fraction plane: dword k (0..6) of lane l at 1024 + 4 (64 k + l): the */
/*       lane's 32 fractions concatenated least significant bit first,      */
/*       fraction j at bit 7 j of the lane's 224-bit string                 */
/*   n_blocks x u32: index of each block's first escape in the list         */
/*   the escape list: u16 symbols in weight order; the whole padded to 16 B */
/* ======================================================================== */
#define BSF_HDR 96u
#define BSF_BLOCK 2048u
#define BSF_BLOCK_BYTES 2816u

/* the up to 15 most frequent symbols, count descending, ties to the lower s */
static uint32_t fixed_table(const uint64_t* cs, uint32_t* tab) {
    uint32_t m = 0;
    int used[512] = {0};
    while (m < 15) {
        int best = -1;
        for (int s = 0; s < 512; s++)
            if (!used[s] && cs[s] && (best < 0 || cs[s] > cs[best])) best = s;
        if (best < 0) break;
        used[best] = 1;
        tab[m++] = (uint32_t)best;
    }
    return m;
}

int bso_fixed_encode(const uint16_t* w, uint64_t n, uint8_t** out, uint64_t* out_len) {
    uint64_t* cs = (uint64_t*)calloc(512, sizeof(uint64_t));
    uint64_t* cf = (uint64_t*)calloc(512 * 128, sizeof(uint64_t));
    if (!cs || !cf) { free(cs); free(cf); return BSO_ENOMEM; }
    bso_histogram(w, n, cs, cf);
    uint32_t tab[16] = {0};
    uint32_t m = fixed_table(cs, tab);
    int code_of[512];
    for (int s = 0; s < 512; s++) code_of[s] = 15;
    for (uint32_t i = 0; i < m; i++) code_of[tab[i]] = (int)i;
    uint64_t n_blocks = (n + BSF_BLOCK - 1) / BSF_BLOCK, n_esc = 0;
    for (uint64_t j = 0; j < n; j++) n_esc += code_of[bso_symbol_s(w[j])] == 15;
    uint64_t offs = BSF_HDR + BSF_BLOCK_BYTES * n_blocks;
    uint64_t esc_off = offs + 4 * n_blocks;
    uint64_t len = round_up(esc_off + 2 * n_esc, 16);
    uint8_t* b = (uint8_t*)calloc(len ? len : 1, 1);
    if (!b) { free(cs); free(cf); return BSO_ENOMEM; }
    memcpy(b, "BF16FIX1", 8);
    put32(b + 8, 1);
    put64(b + 16, n); put64(b + 24, n_blocks); put64(b + 32, esc_off); put64(b + 40, n_esc);
    for (uint32_t i = 0; i < 16; i++) put16(b + 64 + 2 * i, i < m ? tab[i] : 0);
    uint64_t e = 0;
    for (uint64_t blk = 0; blk < n_blocks; blk++) {
        uint8_t* base = b + BSF_HDR + BSF_BLOCK_BYTES * blk;
        put32(b + offs + 4 * blk, (uint32_t)e);
        for (uint32_t l = 0; l < 64; l++) {
            uint64_t j0 = blk * BSF_BLOCK + 32ull * l;
            uint8_t frac[28] = {0};
            for (uint32_t i = 0; i < 32; i++) {
                uint64_t j = j0 + i;
                uint32_t code = 0, f = 0;
                if (j < n) {
                    uint32_t s = bso_symbol_s(w[j]);
                    code = (uint32_t)code_of[s];
                    f = bso_symbol_f(w[j]);
                    if (code == 15) { put16(b + esc_off + 2 * e, s); e++; }
                }
                uint8_t* cw = base + 4 * (64 * (i / 8) + l);
                cw[(i % 8) / 2] |= (uint8_t)(code << (4 * (i % 2)));
                put_bits(frac, 7ull * i, f, 7);
            }
            for (uint32_t k = 0; k < 7; k++)
                for (uint32_t y = 0; y < 4; y++) base[1024 + 4 * (64 * k + l) + y] = frac[4 * k + y];
        }
    }
    free(cs); free(cf);
    *out = b; *out_len = len;
    return BSO_OK;
}

int bso_fixed_decode(const uint8_t* b, uint64_t len, uint16_t* out, uint64_t cap) {
    if (len < BSF_HDR || memcmp(b, "BF16FIX1", 8) != 0) return BSO_EFORMAT;
    if (get32(b + 8) != 1) return BSO_EVERSION;
    uint64_t n = get64(b + 16), n_blocks = get64(b + 24), esc_off = get64(b + 32), n_esc = get64(b + 40);
    if (n_blocks != (n + BSF_BLOCK - 1) / BSF_BLOCK || n_blocks > len / BSF_BLOCK_BYTES) return BSO_EFORMAT;
    uint64_t offs = BSF_HDR + BSF_BLOCK_BYTES * n_blocks;
    if (esc_off != offs + 4 * n_blocks || esc_off + 2 * n_esc > len) return BSO_EFORMAT;
    if (n > cap) return BSO_ENOSPACE;
    uint32_t tab[16];
    for (uint32_t i = 0; i < 16; i++) tab[i] = get16(b + 64 + 2 * i);
    for (uint64_t blk = 0; blk < n_blocks; blk++) {
        const uint8_t* base = b + BSF_HDR + BSF_BLOCK_BYTES * blk;
        uint64_t e = get32(b + offs + 4 * blk);
        for (uint32_t l = 0; l < 64; l++) {
            uint8_t frac[28];
            for (uint32_t k = 0; k < 7; k++)
                for (uint32_t y = 0; y < 4; y++) frac[4 * k + y] = base[1024 + 4 * (64 * k + l) + y];
            for (uint32_t i = 0; i < 32; i++) {
                uint64_t j = blk * BSF_BLOCK + 32ull * l + i;
                if (j >= n) continue;
                uint32_t code = (base[4 * (64 * (i / 8) + l) + (i % 8) / 2] >> (4 * (i % 2))) & 15u;
                uint32_t s;
                if (code == 15) {
                    if (e >= n_esc) return BSO_ECORRUPT;
                    s = get16(b + esc_off + 2 * e);
                    e++;
                    if (s >= 512) return BSO_ECORRUPT;
                } else {
                    s = tab[code];
                }
                out[j] = bso_combine(s, get_bits(frac, 7ull * i, 7));
            }
        }
        /* the block used exactly the escapes up to the next block's first */
        if (e != (blk + 1 < n_blocks ? get32(b + offs + 4 * (blk + 1)) : n_esc)) return BSO_ECORRUPT;
    }
    return BSO_OK;
}
