/*
 * bs.h -- C ABI of the MI355X (gfx950) lossless BF16 weight codec.
 *
 * What the library computes [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec
 * paragraph after the metrics table]: every BF16 word is split into its exact
 * fields [sign:1 | exponent:8 | fraction:7]; the joint 9-bit (sign, exponent)
 * symbol s is coded with a per-tensor rANS model; the decoded s selects the
 * distribution of the exact 7-bit fraction f; decoding recombines the fields
 * bitwise (w = s << 7 | f); spans that are not BF16 pass through verbatim.
 * Every tensor carries a hash checked after decompression [Gemma 2 9B
 * Instruct -- Lossless Compressed card, "What lossless means"; NVLC card,
 * SHA256SUMS verification block] (sha256 here).
 *
 * Container ("BF16RANS", version 1, 2 or 3, little-endian) -- this library's
 * own layout.  Version 1 holds layout-1 records only; version 2 adds layout 2
 * (below) and names each BF16 record's layout in its fixed part; version 3
 * also allows layout 3 (below):
 *   header 64 B: magic[8] "BF16RANS", u32 version, u32 n_records,
 *                u64 dir_offset, u64 total_len, u64 out_len, u32 flags, 20 B zero
 *   directory, 96 B per record: u32 kind (1 = BF16 rANS, 2 = RAW verbatim),
 *                u32 0, u64 n (weights for BF16, bytes for RAW), u64 out_offset,
 *                u64 rec_offset, u64 rec_len, u8 sha256[32], 24 B zero
 *   BF16 record body: u32 W (weights per chunk), u32 K (lanes), u32 n_chunks,
 *                u8 M_s, u8 M_f, u8 n_tables, u8 log2 S (word streams per
 *                chunk), u32 n_sym, u32 layout (version 1: 0, meaning layout
 *                1; version 2: 1 or 2; version 3: 1, 2 or 3); the rest of a layout-1 body:
 *                s-table n_sym x (u16 s, u16 q) ascending s (sum q = 2^M_s);
 *                route: n_sym bytes (fraction table of each s: 0 = flat,
 *                1..n_tables), padded to 4 B; n_tables x 128 x u16 q_f
 *                (each sums to 2^M_f); pad to 16 B; chunk index n_chunks x
 *                (u64 payload offset from the body start, u32 16-bit units
 *                of the chunk's stream area, u32 0); when S > 1 the stream
 *                table n_chunks x (S - 1) x u32: the start unit of streams
 *                1 .. S-1 in the chunk's stream area; pad to 16 B; payloads,
 *                each 16-B aligned: the K lanes' length codes (a nibble per
 *                lane, lane l in the low nibble of byte l/2 when l is even;
 *                pad 16 B), then the stream area: the S streams back to back,
 *                each the state bits of its P lanes (below), padded to a
 *                16-bit unit, followed by its 16-bit words in decode order;
 *                the payload is padded to 16 B.
 *   Final lane states: a state x in [2^16, 2^32) is its length code
 *   e = floor(log2 x) - 16 and its 16 + e bits below the leading one, the
 *   stream's lanes' bits concatenated in lane order, least significant first.
 *   Coder: 32-bit state in [2^16, 2^32), 16-bit renormalisation words.  In a
 *   chunk, weight j belongs to lane (j/8) mod K, macro-step (j/8)/K; each lane
 *   decodes, per weight, s with the s-table then f with the table route[s];
 *   the K lanes form S streams of P = K/S consecutive lanes, each with its
 *   own word sequence; within a stream, lanes take turns in ascending order
 *   in each (macro-step, position, field) sub-step, consuming its words in
 *   that order.  A lane's last group holds c = min(8, weights left) weights;
 *   the last m = min(4, c) of them carry only s in the stream: their
 *   fractions are the low 7m bits of the lane's start state (first of them
 *   lowest) under a leading one at bit max(16, 7m), so the decoder reads them
 *   off the state it ends in.  A lane without weights starts and ends at
 *   2^16.  Fraction tables with id 0 are flat (q = 2^(M_f - 7) for every f).
 *
 * Layout 2 (one renormalisation per weight): the fraction f = h << 4 | l is
 * split into its high three bits h, coded with the distribution s selects,
 * and its low four bits l, stored verbatim.  Per weight a lane decodes s
 * (precision M_s, 11 or 12) and then h (precision M_h = 16 - M_s, held in
 * the M_f byte) with the table route[s], and only then renormalises: the two
 * steps use at most 16 bits of the state, so one 16-bit word restores it.
 * Body after the fixed part: the s-table and route bytes as in layout 1
 * (padded to 4 B), then n_tables (<= 31) x 8 x u8 q_h (each sums to 2^M_h;
 * table 0 is flat, q_h = 2^(M_h - 3)), padded to 16 B; chunk index and stream
 * table as in layout 1.  A chunk payload is the length codes (padded to
 * 16 B), then the plane of low bits, one u32 per group of 8 weights (group g
 * at byte 4 g, padded to 16 B; the l of position p of a group at bit
 * 16 (p mod 2) + 4 (p div 2), 0 past the chunk's end), then the stream area
 * as in layout 1 (its units counted in the chunk index).  Sub-steps are one
 * per weight, (macro-step, position), lanes ascending inside each.  In its
 * last group (c = min(8, weights left) weights) a lane decodes s only: the h
 * of those c weights are the low 3c bits of its start state (first weight
 * lowest) under a leading one at bit max(16, 3c).  A table id > 0 is given to
 * an exponent (both signs share it) when quantising its h counts saves more
 * than 64 bits against the flat table, counted with floor(65536 log2 q);
 * at most max_tables of them, the largest savings first (lower exponent on
 * ties), ids in ascending exponent order.  Every other occupied exponent is
 * routed to the table, flat or coded, that codes its h counts in the fewest
 * bits (sum of m[h] (65536 M_h - floor(65536 log2 q[h])); a table with q = 0
 * for a used h is excluded; the lower id wins ties), so tables are shared
 * between contexts [NVLC card, codec paragraph: "soft-routed fraction
 * distribution", read as a route to a shared table].
 *
 * Layout 3 (one joint symbol per weight): as layout 2, except that outside
 * a lane's last group s and h are coded as one symbol t = 8 s + h with a
 * per-tensor table of precision M_t = 13 (held in the M_f byte; n_tables 0):
 * one coding step and one renormalisation check per weight.  Each s thus
 * has its own h distribution [NVLC card, codec paragraph: the decoded
 * symbol selects the fraction's distribution].  Body after the fixed part:
 * the s-table and route bytes (all 0) as in layout 1, padded to 4 B, then
 * n_sym x 8 x u16 q_t, the joint frequencies of (s, h = 0..7) for each s of
 * the s-table in its order (all summing to 2^13), padded to 16 B; chunk
 * index, stream table, payloads (with the plane), sub-steps and the last
 * group (s alone, h in the start state) as in layout 2.  Frequencies (the
 * s-table's and the joint table's) quantise counts c of n words to 2^M:
 * q = max(1, floor(c 2^M / n)) for c > 0; a shortfall is added one by one
 * in order of the remainder (c 2^M mod n) descending, lower index first,
 * cycling; an excess is taken one at a time from the largest q > 1, lower
 * index first.
 *
 * Conventions:
 *   - Every function returns a bs_status (0 = BS_OK); none throws or aborts.
 *     bs_last_error() gives a thread-local message for the last failure.
 *   - "d_" pointers are device (HBM) pointers, "h_" pointers host pointers.
 *     All tensors and output buffers are caller-owned.  The library owns only
 *     the opaque objects it returns (bs_tables, bs_blob, bs_plan) and frees
 *     them in the matching *_free / *_destroy call.
 *   - Device work is enqueued on the caller's stream (hipStream_t passed as
 *     void*; NULL = the null stream) and is stream-ordered.
 */
#ifndef BS_H
#define BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BS_OK = 0,
    BS_E_INVAL = -1,       /* bad argument */
    BS_E_FORMAT = -2,      /* container malformed or truncated */
    BS_E_VERSION = -3,     /* container version not supported */
    BS_E_NOSPACE = -4,     /* output capacity too small */
    BS_E_NOMEM = -5,       /* host or device allocation failed */
    BS_E_HIP = -6,         /* HIP runtime error */
    BS_E_CORRUPT = -7,     /* decoded data failed its per-chunk checks */
    BS_E_MISMATCH = -8,    /* decoded bytes differ from the reference or digest */
    BS_E_EXISTS = -9       /* refusing to overwrite existing output */
} bs_status;

enum { BS_KIND_BF16 = 1, BS_KIND_RAW = 2 };

/* Encoder parameters.  chunk_weights W must be a multiple of 8*lanes; lanes K
 * is a power of two: 1..64, 128, 256, 512, 1024 or 2048; stream_lanes P
 * (0 = K) is a power of two <= K and <= 512: each chunk's lanes are split into
 * word streams of P lanes (fewer when a small record gets fewer lanes), which
 * the decoder runs on separate wavefronts; threads = host encoder threads
 * (0 = hardware count).  layout 1: 9 <= m_s <= 12, 8 <= m_f <= 10 (the
 * decoder multiplies x >> m in 24 bits, so m >= 8), max_tables <= 6; the
 * container is version 1.  layout 2: m_s 11 or 12, m_f = 16 - m_s (the
 * precision of the h tables), max_tables <= 31; the container is version 2,
 * and the GPU decode takes at most 256 lanes per word stream.  layout 3: m_s
 * 11 or 12, m_f = 13 (the joint table's precision), max_tables unused; the
 * container is version 3, at most 256 lanes per word stream as in layout 2. */
typedef struct {
    uint32_t chunk_weights;
    uint32_t lanes;
    uint32_t m_s;
    uint32_t m_f;
    uint32_t max_tables;
    uint32_t threads;
    uint32_t stream_lanes;
    uint32_t layout;
} bs_params;

/* Fill *p with the defaults: W = 65536, K = 128, layout 3 (the joint
 * (s, h) symbol) with m_s = 11 and m_f = 13 (the joint table's precision),
 * max_tables = 31 (layout 2's coded h tables; layout 3 has none), threads =
 * 0, stream_lanes = 0 (one stream per chunk).  Switching to layout 2 also
 * needs m_f = 16 - m_s; layout 1 takes m_f 8..10 and max_tables <= 6. */
void bs_params_default(bs_params* p);

/* ---------------------------------------------------------------- model */

typedef struct bs_tables bs_tables; /* opaque, library-owned */

/* Build the per-tensor model of n BF16 words that are resident on the device
 * [NVLC card, codec paragraph: the sign/exponent model is per tensor, the
 * fraction distribution is selected by the decoded symbol].
 * One HIP histogram pass with LDS-privatised counters (fraction counts per
 * exponent over both signs, and negative words per exponent and high
 * fraction bits), then host quantisation of the counts to 2^m_s and 2^m_f
 * (layout 3: of the joint counts to 2^13) and the choice of coded fraction
 * contexts.
 * d_bf16: n little-endian 16-bit words in device memory (any alignment of 2).
 * Synchronises `stream`.  *out receives a new bs_tables (free with
 * bs_tables_free).  Errors: BS_E_INVAL (bad params / NULL), BS_E_HIP,
 * BS_E_NOMEM. */
bs_status bs_build_tables(const void* d_bf16, uint64_t n, const bs_params* p, void* stream, bs_tables** out);

/* Same model from host memory (CPU histogram); identical result. */
bs_status bs_build_tables_host(const uint16_t* h_bf16, uint64_t n, const bs_params* p, bs_tables** out);

/* For callers that cannot allocate memory (harnesses that forbid hipMalloc,
 * serving loops that must not touch an allocator): bs_build_tables without
 * any allocation.  The model is written over *t, an existing tables object
 * (from bs_build_tables or bs_build_tables_host); the result is the one
 * bs_build_tables gives for the same words and params.  The histogram's
 * counters sit in a fixed device array of the library (278,528 B on each GPU
 * it runs on, held until the process ends; its size does not depend on n),
 * cleared by a kernel at each call.  Calls in one process are serialised by
 * a host lock held from the clear to the read-back, so they never overlap on
 * a GPU; the array keeps the last call's counts.  Synchronises `stream`.
 * n at most BS_NOALLOC_MAX_WEIGHTS (2^36), beyond it BS_E_INVAL with a
 * message.  Errors: BS_E_INVAL (NULL, bad params, n too large), BS_E_HIP. */
#define BS_NOALLOC_MAX_WEIGHTS (1ull << 36)
bs_status bs_build_tables_noalloc(const void* d_bf16, uint64_t n, const bs_params* p, void* stream, bs_tables* t);

void bs_tables_free(bs_tables* t);

/* Read back a model (for inspection and tests).  Arrays are caller-owned:
 * counts_s[512] (u64, may be NULL), q_s[512], route[512] (table id of each s),
 * q_f[6*128] (layout 1: row t-1 = table t); *n_tables, *m_s, *m_f, *n_weights. */
bs_status bs_tables_get(const bs_tables* t, uint64_t* counts_s, uint32_t* q_s, uint32_t* route,
                        uint32_t* q_f, uint32_t* n_tables, uint32_t* m_s, uint32_t* m_f, uint64_t* n_weights);

/* The model's layout (1, 2 or 3) and, for layout 2, its h tables: q_h[31*8]
 * (row t-1 = table t; may be NULL). */
bs_status bs_tables_get_layout(const bs_tables* t, uint32_t* layout, uint32_t* q_h);

/* A layout-3 model's joint table: q_t[4096] receives the frequency of each
 * joint symbol 8 s + h (sum 2^13; zeros for a model of another layout)
 * [NVLC card, codec paragraph: the fraction's distribution is selected by
 * the decoded symbol].  Errors: BS_E_INVAL (NULL). */
bs_status bs_tables_get_joint(const bs_tables* t, uint32_t* q_t);

/* ---------------------------------------------------------------- encode */

/* One tensor to encode.  kind BS_KIND_BF16: h_data holds n 16-bit words and
 * tables is its model (NULL = built on the host here).  kind BS_KIND_RAW:
 * h_data holds n bytes copied verbatim (the residual for non-BF16 spans
 * [NVLC card, codec paragraph]).  sha256: 32 bytes or NULL (computed here). */
typedef struct {
    uint32_t kind;
    uint32_t reserved;
    const void* h_data;
    uint64_t n;
    const bs_tables* tables;
    const uint8_t* sha256;
} bs_tensor;

typedef struct bs_blob bs_blob; /* opaque, library-owned byte buffer */

/* Encode tensors[0..n_tensors) into one container, in order, on host threads
 * [Qwen3.8-27B-BF16-NVLC-Lossless card, codec paragraph after the metrics
 * table: each BF16 word split into its exact fields, the (sign, exponent)
 * symbol rANS-coded with a per-tensor model, the fraction coded with the
 * distribution that symbol selects, a residual for non-BF16 spans; the
 * chunk, lane and byte layout are this library's own (header comment)].
 * Output offsets are assigned in order, each rounded up to 256 B.  A BF16
 * tensor with more than 256 distinct (sign, exponent) symbols is stored as a
 * RAW record of its bytes.  The result is deterministic (independent of the
 * thread count).  *out receives a new bs_blob (free with bs_blob_free).
 * Errors: BS_E_INVAL (bad params, a model built for another n), BS_E_NOMEM. */
bs_status bs_encode_host(const bs_tensor* tensors, uint32_t n_tensors, const bs_params* p, bs_blob** out);

/* --------------------------------------------------------------- GPU encoder
 *
 * The container bs_encode_host writes, byte for byte, built from tensors in
 * device memory: each record's word streams are coded on the GPU, one
 * wavefront per stream, running the decode order backwards (the rANS coding
 * step of the NVLC card's codec paragraph, in this library's chunk, lane and
 * stream layout above).  Three calls: begin codes every stream into
 * library-owned device scratch and lays the container out (it synchronises
 * `stream` once, to read the streams' sizes back); size gives the container's
 * length; finish writes the container into caller memory. */
typedef struct {
    uint32_t kind;              /* BS_KIND_BF16 or BS_KIND_RAW */
    uint32_t reserved;
    const void* d_data;         /* device: n 16-bit words (BF16, 16-B aligned) or n bytes (RAW) */
    uint64_t n;
    const bs_tables* tables;    /* NULL: built here with bs_build_tables */
    const uint8_t* sha256;      /* 32 bytes, or NULL: computed from a host copy (slow) */
} bs_dtensor;

typedef struct bs_dencoder bs_dencoder; /* opaque, library-owned */

/* Errors: BS_E_INVAL (bad params, kind, NULL or misaligned data, a model
 * built for other data), BS_E_NOMEM, BS_E_HIP. */
bs_status bs_encode_device_begin(const bs_dtensor* tensors, uint32_t n_tensors, const bs_params* p, void* stream,
                                 bs_dencoder** out);
uint64_t bs_encode_device_size(const bs_dencoder* e);
/* Write the container (bs_encode_device_size bytes) to d_out (16-B aligned),
 * enqueued on `stream`; the tensors must stay unchanged until it completes.
 * Errors: BS_E_INVAL, BS_E_NOSPACE, BS_E_HIP. */
bs_status bs_encode_device_finish(bs_dencoder* e, void* d_out, uint64_t capacity, void* stream);
/* Waits for the encoder's work, then frees it. */
void bs_encode_device_free(bs_dencoder* e);

const void* bs_blob_data(const bs_blob* b);
uint64_t bs_blob_size(const bs_blob* b);
void bs_blob_free(bs_blob* b);

/* ---------------------------------------------------------------- inspect */

typedef struct {
    uint32_t version;
    uint32_t n_records;
    uint64_t total_len;
    uint64_t out_len;       /* bytes of the fully decoded output */
    uint64_t n_chunks;      /* chunks over all BF16 records */
    uint64_t bf16_weights;  /* BF16 weights over all BF16 records */
    uint64_t bf16_bytes;    /* container bytes charged to BF16 records (bodies + their directory share + header share) */
    uint64_t raw_bytes;     /* verbatim bytes */
    uint64_t n_streams;     /* word streams over all BF16 chunks (status array length) */
} bs_container_info;

typedef struct {
    uint32_t kind;
    uint32_t chunk_weights, lanes, n_chunks;
    uint32_t m_s, m_f, n_tables, n_sym;
    uint64_t n, out_offset, rec_offset, rec_len;
    uint64_t chunk_base;    /* index of the record's first chunk over all BF16 records */
    uint8_t sha256[32];
    uint64_t stream_base;   /* status index of the record's first stream */
    uint32_t streams;       /* word streams per chunk */
    uint32_t layout;        /* BF16 records: 1, 2 or 3 */
} bs_record_info;

/* Where a container's BF16 bits go [Qwen3.8-27B-BF16-NVLC-Lossless card,
 * metrics table: its bits per weight count every byte of the compressed
 * checkpoint against the weights it holds]: in bits, over all
 * its BF16 records, summing exactly to 8 x bs_container_info.bf16_bytes (all
 * zero when the container holds no BF16 weights). */
typedef struct {
    uint64_t weights;         /* BF16 weights */
    uint64_t container_bits;  /* the BF16 side's share of the header, directory and gaps between records */
    uint64_t fixed_bits;      /* record bodies' fixed parts (24 B each) */
    uint64_t table_bits;      /* s-tables, routes, fraction / h / joint tables, their padding */
    uint64_t index_bits;      /* chunk index and stream table, padded up to the first payload */
    uint64_t code_bits;       /* the lanes' length codes, padded to 16 B per chunk */
    uint64_t plane_bits;      /* layouts 2 and 3: the verbatim low fraction bits, padded to 16 B per chunk */
    uint64_t state_bits;      /* final lane states: 16 + e bits each */
    uint64_t word_bits;       /* the streams' 16-bit words */
    uint64_t pad_bits;        /* the rest of the records: state bits padded to 16-bit units, payloads to 16 B */
} bs_size_breakdown;

/* Validate a host copy of a container and describe it.  Errors: BS_E_FORMAT,
 * BS_E_VERSION. */
bs_status bs_container_info_get(const void* h_container, uint64_t len, bs_container_info* info);
bs_status bs_record_info_get(const void* h_container, uint64_t len, uint32_t index, bs_record_info* info);
/* The size breakdown of a host copy of a container (validated as above).
 * Errors: BS_E_INVAL (NULL), BS_E_FORMAT, BS_E_VERSION. */
bs_status bs_container_sizes_get(const void* h_container, uint64_t len, bs_size_breakdown* out);

/* ---------------------------------------------------------------- decode */

typedef struct bs_plan bs_plan; /* opaque, library-owned device work list + lookup tables */

/* Prepare decoding of a container resident in device memory.  h_container is
 * a host copy of the same bytes (only its header, directory, tables and chunk
 * index are read); d_container the device copy (len bytes, 16-B aligned).
 * Validates everything the kernels rely on (record bounds, table sums, chunk
 * payload bounds), allocates the plan's device memory, uploads the work list
 * and builds each record's decode lookup tables with a HIP kernel on
 * `stream`.  The plan references d_container, which must stay valid and
 * unchanged while the plan is used.  Errors: BS_E_FORMAT, BS_E_VERSION,
 * BS_E_NOMEM, BS_E_HIP. */
bs_status bs_plan_create(const void* h_container, uint64_t len, const void* d_container, void* stream,
                         bs_plan** out);
void bs_plan_destroy(bs_plan* plan);

/* Point a plan at another device copy of the same container bytes (d_container,
 * 16-B aligned), for containers that move between device buffers (the layer
 * streamer below).  Work enqueued before the call keeps the old address.
 * Errors: BS_E_INVAL. */
bs_status bs_plan_rebind(bs_plan* plan, const void* d_container);

/* Length in bytes of the plan's container. */
uint64_t bs_plan_container_bytes(const bs_plan* plan);

/* Decode records [first, first + count) into d_out, enqueued on `stream`
 * (no host synchronisation) [Qwen3.8-27B-BF16-NVLC-Lossless card, codec
 * paragraph: the (sign, exponent) symbol is decoded first, it selects the
 * fraction's distribution, and the fields are recombined bitwise into the
 * original word; non-BF16 spans come back verbatim from the residual].  Record i is written at
 * d_out + out_offset(i) - out_offset(first); the bytes between records are not
 * written.  d_out must be 16-B aligned with at least the returned
 * bs_plan_out_bytes(plan, first, count) bytes of capacity; nothing outside
 * [d_out, d_out + that size) is written.  d_status: one u32 per word stream
 * of the whole container (bs_container_info.n_streams; stream s of chunk c of
 * a record at stream_base + c * streams + s); the entries of the decoded
 * records are set to 0 (ok) or a bit set: 1 = a lane did not end at the
 * initial state, 2 = the words consumed differ from the stream's count.  The
 * output is valid after the stream reaches this point.  Errors (returned
 * before anything is enqueued): BS_E_INVAL (range, alignment), BS_E_NOSPACE
 * (out_capacity too small), BS_E_HIP (launch failed). */
bs_status bs_decode_async(const bs_plan* plan, uint32_t first, uint32_t count, void* d_out, uint64_t out_capacity,
                          uint32_t* d_status, void* stream);

/* Fused decode and matrix-vector product [Qwen3.8-27B-BF16-NVLC-Lossless
 * card, runtime paragraphs: the compressed-only runtime decodes weights where
 * they are used and keeps no decoded copy]: y[r] = sum over c of W[r, c] x[c]
 * for BF16 record `record` read as a row-major rows x cols matrix
 * (rows * cols = its weight count; cols a multiple of 8 and at least 512).
 * The weights are decoded in registers and never written out.  d_x: cols
 * BF16 words, 16-B aligned; d_y: rows floats, overwritten (a fill kernel
 * clears it first, then the products are added in fp32, in an order that
 * varies from run to run, so the result matches the exact sum within the
 * usual fp32 summation bound, not bit for bit).  d_status as for
 * bs_decode_async (only the record's entries are written).  Records of
 * either layout are accepted; layout-1 records in the compact table layout
 * or with more than 4 lanes per thread are rejected (BS_E_INVAL).  Enqueued
 * on `stream`; nothing is allocated. */
bs_status bs_gemv_async(const bs_plan* plan, uint32_t record, uint64_t rows, uint64_t cols, const void* d_x, float* d_y,
                        uint32_t* d_status, void* stream);

/* -------------------------------------------------- fixed-width lane streams
 *
 * A second device form of one BF16 tensor, derived from it once and decoded
 * without any sequential chain [NVLC card, runtime paragraphs and runtime
 * accounting table: the measured GPU runtime derives fixed-width,
 * lane-oriented streams (the Fixed7/Compact11 runtime) from the canonical
 * model at initialisation, about 71% of the raw BF16 bytes resident; the
 * layout below is this library's own].  Every weight is an 11-bit code
 * word: a 4-bit code naming one of the tensor's 15 most frequent
 * (sign, exponent) symbols, or 15 = escape, and the exact 7-bit fraction.
 * Layout (all integers little-endian):
 *   header, 96 B: "BF16FIX1", u32 version (1), u32 0, u64 n (weights),
 *     u64 n_blocks = ceil(n / 2048), u64 esc_off, u64 n_esc, 16 B zero,
 *     16 x u16: the symbol of codes 0..14 in order of count (descending,
 *     ties to the lower symbol; 0 where fewer than 15 occur), entry 15 = 0
 *   n_blocks blocks of 2816 B from byte 96; lane l (0..63) of block b holds
 *     weights 2048 b + 32 l .. + 31 (past n: code 0, fraction 0):
 *     code plane: dword k (0..3) of lane l at +4 (64 k + l), the code of the
 *       lane's weight 8 k + i in bits 4 i .. 4 i + 3;
 *     fraction plane: dword k (0..6) of lane l at +1024 + 4 (64 k + l): the
 *       lane's 32 fractions, weight i at bit 7 i of the 224 bits these seven
 *       dwords hold (least significant first)
 *   n_blocks x u32 from 96 + 2816 n_blocks: index of each block's first
 *     escape in the escape list
 *   the escape list at esc_off = 96 + 2820 n_blocks: n_esc u16 symbols, one
 *     per code 15, in weight order; the blob is zero-padded to 16 B. */
typedef struct {
    uint64_t n;             /* weights */
    uint64_t n_blocks;
    uint64_t n_esc;         /* escaped weights */
    uint64_t esc_off;       /* byte offset of the escape list */
    uint64_t bytes;         /* blob length */
    uint16_t table[16];     /* symbol of codes 0..14; entry 15 = 0 */
} bs_fixed_info;

/* Fixed-width form of h_words[0..n) (host), built on up to `threads` host
 * threads (0 = all); deterministic.  *out receives a new bs_blob.  Errors:
 * BS_E_INVAL (NULL), BS_E_NOMEM. */
bs_status bs_fixed_encode_host(const uint16_t* h_words, uint64_t n, uint32_t threads, bs_blob** out);

/* Largest fixed-width blob of n weights (every weight an escape). */
uint64_t bs_fixed_max_bytes(uint64_t n);

/* The same blob as bs_fixed_encode_host, built on the GPU from n BF16 words in
 * device memory (d_words, 16-B aligned) into d_out (16-B aligned, capacity
 * bytes): a symbol-count kernel, the table on the host, an escape-count
 * kernel per block, the block offsets on the host, then a pack kernel (one
 * wavefront per block).  *out_len receives the blob's length (also when the
 * capacity is too small; bs_fixed_max_bytes(n) always suffices).  Meant for
 * initialisation: it allocates device scratch and synchronises `stream`.
 * Errors: BS_E_INVAL, BS_E_NOSPACE, BS_E_NOMEM, BS_E_HIP. */
bs_status bs_fixed_encode_device(const void* d_words, uint64_t n, void* d_out, uint64_t capacity, uint64_t* out_len,
                                 void* stream);

/* Validate the header of a fixed-width blob and describe it.  h_header: a
 * host copy of at least its first 96 bytes (header_len of them readable);
 * blob_len: the whole blob's length.  Checks the magic, version, block count,
 * escape list offset and that the escape list fits in blob_len; symbols
 * above 511 in the table are a format error.  Errors: BS_E_INVAL,
 * BS_E_FORMAT, BS_E_VERSION. */
bs_status bs_fixed_info_get(const void* h_header, uint64_t header_len, uint64_t blob_len, bs_fixed_info* info);

/* Decode a fixed-width blob resident in device memory (d_blob, info->bytes
 * bytes, 16-B aligned; `info` from bs_fixed_info_get on the same bytes) into
 * d_out (info->n BF16 words, 16-B aligned, at least 2 n bytes of capacity;
 * nothing else is written).  d_status: NULL, or info->n_blocks u32, each set
 * to 0 (ok) or a bit set: 1 = the block's codes hold another number of
 * escapes than its escape range, 2 = its escape range is out of order or
 * beyond n_esc, 4 = an escape symbol above 511.  Escaped weights that such a
 * block cannot resolve get symbol 0.  Enqueued on `stream`; nothing is
 * allocated.  Errors (before anything is enqueued): BS_E_INVAL (NULL,
 * alignment), BS_E_NOSPACE, BS_E_HIP. */
bs_status bs_fixed_decode_async(const bs_fixed_info* info, const void* d_blob, void* d_out, uint64_t out_capacity,
                                uint32_t* d_status, void* stream);

/* Decode up to BS_FIXED_MANY_MAX fixed-width blobs in one kernel launch (a
 * layer's tensors, say): blob i as bs_fixed_decode_async(&infos[i],
 * d_blobs[i], d_outs[i], out_capacities[i], d_status ? d_status[i] : NULL).
 * The launch's workgroups are shared among the blobs in proportion to their
 * blocks (at least one each), so the blobs decode side by side and the
 * launch ends once, with no tail per tensor.  Blobs with n = 0 are skipped;
 * outputs must not overlap.  Every argument is checked before anything is
 * enqueued.  Errors: BS_E_INVAL (count above BS_FIXED_MANY_MAX, NULL,
 * alignment, an info not from bs_fixed_info_get), BS_E_NOSPACE, BS_E_HIP. */
#define BS_FIXED_MANY_MAX 16
bs_status bs_fixed_decode_many_async(const bs_fixed_info* infos, const void* const* d_blobs, void* const* d_outs,
                                     const uint64_t* out_capacities, uint32_t* const* d_status, uint32_t count,
                                     void* stream);

/* Fused decode and matrix-vector product on a fixed-width blob [NVLC card,
 * runtime paragraphs: the compressed-only runtime multiplies with weights
 * decoded where they are used and keeps no decoded copy]: y[r] = sum over c
 * of W[r, c] x[c], the blob's n weights read as a row-major rows x cols
 * matrix (rows * cols = n, cols a multiple of 32 and below 2^26).  The
 * weights are decoded in registers and never written out.  d_x: cols BF16
 * words, 16-B aligned; d_y: rows floats, overwritten.  One workgroup owns
 * whole rows, so the products of a row are summed in fp32 in one fixed order:
 * the result is the same on every run and matches the exact sum within the
 * usual fp32 summation bound (not bit for bit).  d_status as for
 * bs_fixed_decode_async.  One kernel launch on `stream`; nothing is
 * allocated.  Errors: BS_E_INVAL (shape, NULL, alignment), BS_E_HIP. */
bs_status bs_fixed_gemv_async(const bs_fixed_info* info, const void* d_blob, uint64_t rows, uint64_t cols,
                              const void* d_x, float* d_y, uint32_t* d_status, void* stream);

/* Fused decode and product with a batch of vectors on the matrix cores
 * [NVLC card, runtime paragraphs: the compressed-only runtime multiplies with
 * weights decoded where they are used]: Y[b, r] = sum over c of W[r, c] X[b, c]
 * for b < batch (1..64), with W the blob's n weights as a row-major rows x cols
 * matrix, cols a multiple of 2048 (so every row starts on a block) and below
 * 2^26, rows below 2^26.  A workgroup decodes its rows a panel of 2048 columns at a time into
 * LDS and multiplies them with v_mfma_f32_16x16x32_bf16; the weights are
 * never written out.  d_x: batch x cols BF16 words, row-major, 16-B aligned;
 * d_y: batch x rows floats, row-major, overwritten.  d_status as for
 * bs_fixed_decode_async.
 *
 * Without a workspace (d_work NULL) a workgroup owns 16 rows and all their
 * panels: one launch, nothing allocated.  With one (cols >= 4096), a
 * workgroup takes 32 rows, so that each element of X it reads serves twice
 * the rows, and half of their panels; the other half goes to a second
 * workgroup, which leaves its partial sums in the workspace, and a second
 * launch on `stream` adds them into Y.  d_work: 256-B aligned, work_bytes at
 * least 4 * batch * rows (bs_fixed_gemm_work_bytes gives that size where a
 * workspace helps); its contents need no initialisation and are overwritten.
 * Calls that share a workspace must not overlap (enqueue them on one stream).
 * Either way every entry is summed in fp32 in one fixed order: the same
 * result on every run, within the fp32 summation bound of the exact sum.
 * Errors: BS_E_INVAL (shape, batch, NULL, alignment, a workspace too small
 * or overlapping Y), BS_E_HIP. */
bs_status bs_fixed_gemm_async(const bs_fixed_info* info, const void* d_blob, uint64_t rows, uint64_t cols,
                              uint32_t batch, const void* d_x, float* d_y, uint32_t* d_status, void* d_work,
                              uint64_t work_bytes, void* stream);

/* The workspace that bs_fixed_gemm_async should be given for this shape, in
 * bytes, or 0 where the product runs best without one (batch below 8, a
 * single panel, or a shape it refuses) [the product of the NVLC card's
 * runtime paragraphs, as for bs_fixed_gemm_async]. */
uint64_t bs_fixed_gemm_work_bytes(uint64_t rows, uint64_t cols, uint32_t batch);

/* Bytes needed to decode records [first, first + count). */
uint64_t bs_plan_out_bytes(const bs_plan* plan, uint32_t first, uint32_t count);

/* Wavefronts per decode workgroup when the whole container is decoded (one
 * word stream of a chunk per wavefront at a time). */
uint32_t bs_plan_waves_per_block(const bs_plan* plan);

/* Workgroups of bs_decode_async(plan, first, count, ...) that decode packs of
 * small records (0: none).  In a launch that also holds large records
 * (layouts 2 and 3), records of at most one round of a workgroup's waves are
 * decoded several to a workgroup, one after another, so that they do not
 * each hold a CU for the whole launch; the pack size keeps a pack's decode
 * well below a large run's.  For tests and tuning; 0 for a NULL plan or a
 * range out of bounds. */
uint32_t bs_plan_packs(const bs_plan* plan, uint32_t first, uint32_t count);

/* ------------------------------------------------------- layer streaming
 *
 * Layers streamed on demand under a budget of device memory [Gemma 2 9B
 * Instruct -- Lossless Compressed card, "Low-VRAM streaming": layers are
 * streamed on demand, with an LRU bound on the device memory they use].  A
 * streamer keeps a model's containers (one per layer) in pinned host memory.
 * A layer that is not resident is copied to a device staging buffer on the
 * streamer's own copy stream (so the copy overlaps the caller's work) and
 * decoded on the caller's stream into one of a fixed set of device slots,
 * replacing the least recently used layer that is not acquired.  Every
 * device buffer (slots, two staging buffers, one plan per layer) is
 * allocated when the streamer is created; acquiring, prefetching and
 * releasing allocate nothing.  Not thread-safe: one host thread drives a
 * streamer. */
typedef struct bs_streamer bs_streamer; /* opaque, library-owned */

typedef struct {
    uint32_t n_layers;
    uint32_t n_slots;           /* decoded layers that fit the budget */
    uint64_t slot_bytes;        /* the largest decoded layer, rounded to 256 B */
    uint64_t staging_bytes;     /* each of the two staging buffers */
    uint64_t plan_bytes;        /* device memory of the layers' plans (tables, descriptors) */
    uint64_t hits, misses, evictions;
    uint64_t h2d_bytes;         /* container bytes copied host -> device */
} bs_streamer_stats;

/* Create a streamer for n_layers containers (h_containers[i], lens[i] bytes;
 * host memory, copied into the streamer's pinned memory).  vram_budget bounds
 * the decoded slots plus the two staging buffers; at least two slots must
 * fit.  Each layer's plan is built here (its container passes through a
 * staging buffer once, on `stream`, which is synchronised).  Errors:
 * BS_E_INVAL (NULL, no layers, budget below two slots), BS_E_FORMAT,
 * BS_E_VERSION (a container), BS_E_NOMEM, BS_E_HIP. */
bs_status bs_streamer_create(const void* const* h_containers, const uint64_t* lens, uint32_t n_layers,
                             uint64_t vram_budget, void* stream, bs_streamer** out);
void bs_streamer_destroy(bs_streamer* s);

/* Make layer `layer` resident and acquired; *d_layer receives its decoded
 * bytes (laid out as bs_decode_async of all its records), valid for work
 * enqueued on `stream` after this call until bs_streamer_release.  A miss
 * enqueues the copy on the copy stream and the decode on `stream`; a hit on a
 * layer decoded on another stream makes `stream` wait for that decode.
 * Errors: BS_E_INVAL (layer out of range), BS_E_NOSPACE (every slot is
 * acquired), BS_E_HIP. */
bs_status bs_streamer_acquire(bs_streamer* s, uint32_t layer, void* stream, void** d_layer);

/* Release an acquired layer: work enqueued on `stream` before this call is
 * the last that reads it, and its slot may be reused after that work.
 * Errors: BS_E_INVAL (not acquired). */
bs_status bs_streamer_release(bs_streamer* s, uint32_t layer, void* stream);

/* Start making `layer` resident without acquiring it (copy on the copy
 * stream, decode on `stream`): a later acquire finds it.  Errors as for
 * acquire. */
bs_status bs_streamer_prefetch(bs_streamer* s, uint32_t layer, void* stream);

bs_status bs_streamer_get_stats(const bs_streamer* s, bs_streamer_stats* stats);

/* ---------------------------------------------------------------- verify */

enum {
    BS_VERIFY_STATUS = 1,   /* read back d_status and report corrupt chunks */
    BS_VERIFY_COMPARE = 2,  /* device byte compare of d_out against d_ref */
    BS_VERIFY_SHA256 = 4    /* copy each record back and compare its sha256 with the directory */
};

typedef struct {
    uint64_t chunks_checked;
    uint64_t chunks_bad;          /* chunks with at least one bad stream status */
    uint64_t first_bad_chunk;     /* chunk index over all BF16 records, UINT64_MAX if none */
    uint64_t bytes_compared;
    uint64_t bytes_mismatched;
    uint64_t first_mismatch;      /* byte offset relative to d_out, UINT64_MAX if none */
    uint32_t records_hashed;
    uint32_t records_hash_bad;
    uint32_t first_hash_bad;      /* record index, UINT32_MAX if none */
    uint32_t reserved;
} bs_report;

/* Synchronise `stream`, then check records [first, first + count) of a
 * decode made with the same plan and range [Gemma 2 9B Instruct -- Lossless
 * Compressed card, "What lossless means": every tensor is hash-checked after
 * decompression; Qwen3.8-27B-BF16-NVLC-Lossless card, metrics table and
 * SHA256SUMS block: per-codec and full inverse verification, sha256
 * digests].  d_ref (BS_VERIFY_COMPARE) holds
 * the expected bytes laid out like d_out.  Returns BS_OK when every requested
 * check passes, BS_E_CORRUPT when a chunk status is bad, BS_E_MISMATCH when
 * bytes or a digest differ; the report is filled in every case.  Errors:
 * BS_E_INVAL, BS_E_HIP, BS_E_NOMEM. */
bs_status bs_verify(const bs_plan* plan, uint32_t first, uint32_t count, const void* d_out, const void* d_ref,
                    const uint32_t* d_status, uint32_t flags, void* stream, bs_report* report);

/* ---------------------------------------------------------------- misc */

/* sha256 of n host bytes (FIPS 180-4), into out[32]. */
void bs_sha256(const void* h_data, uint64_t n, uint8_t out[32]);

/* Write a container to `path`, refusing to replace an existing file
 * (BS_E_EXISTS), as the pages' reconstruction tool refuses an existing
 * output path [NVLC card, reconstruction instructions]. */
bs_status bs_write_file_new(const char* path, const void* h_data, uint64_t n);

const char* bs_strerror(bs_status s);
const char* bs_last_error(void);
const char* bs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BS_H */
