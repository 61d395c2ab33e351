// The extern "C" entry points of librec: host-side argument checks, table
// descriptor preparation, and kernel launches on the caller's stream.  Every
// check runs before the first HIP call, so a rejected call touches no device.
#include <string.h>

#include <mutex>
#include <string>

#include <vector>

#include "rec_internal.h"

using namespace rec;

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_time[REC_TIME_KINDS][2];

rec_status fail(rec_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

rec_status ok() {
    g_err.clear();
    return REC_OK;
}

rec_status hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    return fail(REC_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validate one table and build its kernel descriptor.
rec_status prep_table(const rec_table& t, const char* what, TabDev* out) {
    if (t.kind != REC_DIRECT && t.kind != REC_HASH)
        return fail(REC_EINVAL, std::string(what) + ": unknown kind");
    if (t.dim != REC_DIM) return fail(REC_EINVAL, std::string(what) + ": dim must be 16");
    if (t.rows < 1) return fail(REC_EINVAL, std::string(what) + ": rows must be >= 1");
    if (!t.values) return fail(REC_EINVAL, std::string(what) + ": values is NULL");
    if (!aligned16(t.values)) return fail(REC_EINVAL, std::string(what) + ": values not 16-byte aligned");
    memset(out, 0, sizeof(*out));
    out->values = t.values;
    out->rows = t.rows;
    out->kind = t.kind;
    if (t.kind == REC_HASH) {
        if (!t.keys || !t.digests) return fail(REC_EINVAL, std::string(what) + ": hash table needs keys and digests");
        if (!aligned16(t.digests) || ((uintptr_t)t.keys & 7u))
            return fail(REC_EINVAL, std::string(what) + ": digests must be 16-byte and keys 8-byte aligned");
        if (t.rows > 2147483647LL) return fail(REC_EINVAL, std::string(what) + ": hash capacity above 2^31-1");
        out->keys = t.keys;
        out->digests = t.digests;
    } else {
        floor_mod_prepare(t.rows, &out->magic, &out->shift);
    }
    return REC_OK;
}

int num_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return -1;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    return n;
}

// Checks of rec_din_plan's arguments (messages prefixed with `fn`) and its
// kernel arguments; *work is false when there is nothing to launch.  The
// prep functions make no HIP call (the caller sets `waves` once every check
// has passed).
rec_status prep_plan(const char* fn, const rec_table* seq_tables, const int64_t* seq_values,
                     int64_t seq_stride, const int64_t* seq_offsets, const int32_t* seq_lengths,
                     int64_t B, int32_t max_len, int32_t range_positions, int64_t* seq_offsets_out,
                     int64_t* rows_out, void* plan, size_t plan_bytes, PlanArgs* a, bool* work,
                     const char* buf = "plan", const char* need_fn = "rec_din_plan_bytes") {
    const std::string f(fn);
    *work = false;
    if (B < 0) return fail(REC_EINVAL, f + ": B < 0");
    if (B > REC_MAX_B) return fail(REC_EUNSUPPORTED, f + ": B > REC_MAX_B");
    if (max_len < 1 || max_len > REC_MAX_SEQ_LEN)
        return fail(REC_EINVAL, f + ": max_len outside [1, REC_MAX_SEQ_LEN]");
    if (range_positions != 0 &&
        (range_positions % 16 != 0 || range_positions < kMinRange || range_positions > kMaxRange))
        return fail(REC_EINVAL, f + ": range_positions must be 0 or a multiple of 16 in [16, 2^20]");
    if (!seq_tables) return fail(REC_EINVAL, f + ": seq_tables is NULL");
    if (B > 0 && (!seq_lengths || !seq_values))
        return fail(REC_EINVAL, f + ": seq_lengths and seq_values are required");
    if (seq_stride < 0) return fail(REC_EINVAL, f + ": seq_stride < 0");
    if (!plan) return fail(REC_EWORKSPACE, f + ": " + buf + " is NULL");
    if (!aligned16(plan)) return fail(REC_EINVAL, f + ": " + buf + " not 16-byte aligned");
    if (plan_bytes < rec_din_plan_bytes(B, max_len))
        return fail(REC_EWORKSPACE, f + ": " + buf + " smaller than " + need_fn + "(B, max_len)");
    memset(a, 0, sizeof(*a));
    for (int t = 0; t < 3; ++t) {
        rec_status st = prep_table(seq_tables[t], (f + ": seq table").c_str(), &a->tab[t]);
        if (st != REC_OK) return st;
        if (seq_tables[t].rows > 2147483647LL)
            return fail(REC_EUNSUPPORTED, f + ": sequence tables are limited to 2^31-1 rows");
    }
    if (B == 0) return REC_OK;
    a->seq_values = seq_values;
    a->seq_stride = seq_stride;
    a->seq_offsets = seq_offsets;
    a->seq_lengths = seq_lengths;
    a->B = B;
    a->max_len = max_len;
    a->range_positions = range_positions;
    a->seq_offsets_out = seq_offsets_out;
    a->rows_out = rows_out;
    a->plan = plan;
    *work = true;
    return REC_OK;
}

// The same for rec_din_attn_fwd.
rec_status prep_attn(const char* fn, const rec_table* seq_tables, const void* plan, size_t plan_bytes,
                     int64_t B, int32_t max_len, const float* query, int64_t query_ld,
                     const int32_t* query_col, const rec_din_mlp* mlp, float* out,
                     float* scores_out, float* weights_out, DinArgs* a, bool* work,
                     const char* buf = "plan", const char* need_fn = "rec_din_plan_bytes") {
    const std::string f(fn);
    *work = false;
    if (B < 0) return fail(REC_EINVAL, f + ": B < 0");
    if (B > REC_MAX_B) return fail(REC_EUNSUPPORTED, f + ": B > REC_MAX_B");
    if (max_len < 1 || max_len > REC_MAX_SEQ_LEN)
        return fail(REC_EINVAL, f + ": max_len outside [1, REC_MAX_SEQ_LEN]");
    if (!seq_tables) return fail(REC_EINVAL, f + ": seq_tables is NULL");
    if (!query || !query_col) return fail(REC_EINVAL, f + ": query and query_col are required");
    if (!aligned16(query) || query_ld < 16 || (query_ld & 3))
        return fail(REC_EINVAL, f + ": query rows must be 16-byte aligned (query_ld a multiple of 4)");
    for (int t = 0; t < 3; ++t)
        if (query_col[t] < 0 || (query_col[t] & 3) || query_col[t] + 16 > query_ld)
            return fail(REC_EINVAL, f + ": query_col must be multiples of 4 inside query_ld");
    if (!mlp) return fail(REC_EINVAL, f + ": mlp is NULL");
    if (mlp->dtype != REC_F32 && mlp->dtype != REC_BF16 && mlp->dtype != REC_BF16_PACKED)
        return fail(REC_EINVAL, f + ": unknown mlp dtype");
    const bool packed = mlp->dtype == REC_BF16_PACKED;
    if (!mlp->w1 || !mlp->b1 || (!packed && !mlp->w2) || !mlp->b2 || !mlp->w3)
        return fail(REC_EINVAL, f + ": mlp arrays are required");
    if (!aligned16(mlp->w1) || (!packed && !aligned16(mlp->w2)))
        return fail(REC_EINVAL, f + ": w1/w2 not 16-byte aligned");
    if (!out) return fail(REC_EINVAL, f + ": out is NULL");
    if (!aligned16(out)) return fail(REC_EINVAL, f + ": out not 16-byte aligned");
    if (weights_out && !scores_out)
        return fail(REC_EINVAL, f + ": weights_out requires scores_out");
    if (!plan) return fail(REC_EWORKSPACE, f + ": " + buf + " is NULL");
    if (plan_bytes < rec_din_plan_bytes(B, max_len))
        return fail(REC_EWORKSPACE, f + ": " + buf + " smaller than " + need_fn + "(B, max_len)");
    memset(a, 0, sizeof(*a));
    for (int t = 0; t < 3; ++t) {
        rec_status s = prep_table(seq_tables[t], (f + ": seq table").c_str(), &a->tab[t]);
        if (s != REC_OK) return s;
    }
    if (B == 0) return REC_OK;
    const PlanLayout L = plan_layout(B, max_len);
    const char* p = (const char*)plan;
    a->query = query;
    a->query_ld = query_ld;
    for (int t = 0; t < 3; ++t) a->qcol[t] = query_col[t];
    a->max_len = max_len;
    a->w1 = mlp->w1;
    a->b1 = mlp->b1;
    a->w2 = mlp->w2;
    a->b2 = mlp->b2;
    a->w3 = mlp->w3;
    a->b3 = mlp->b3;
    a->dtype = mlp->dtype;
    a->plan_hdr = (const int32_t*)p;
    a->pos_start = (const int32_t*)(p + L.off_pos);
    a->pos_b = (const int32_t*)(p + L.off_pb);
    a->pos_jr = (const int32_t*)(p + L.off_pjr);
    a->pos_rows = (const int32_t*)(p + L.off_prows);
    a->group_start = (const int32_t*)(p + L.off_group);
    a->ngroups = L.ngroups;
    a->empty = (const int32_t*)(p + L.off_empty);
    a->pmax = L.pmax;
    a->out = out;
    a->scores = scores_out;
    a->weights = weights_out;
    a->B = B;
    *work = true;
    return REC_OK;
}

// Checks of rec_embbag_fwd_kjt's arguments (messages prefixed with `fn`) and
// its kernel arguments; *work is false when there is nothing to launch.
rec_status prep_embbag_kjt(const char* fn, const rec_table* tables, int32_t T, int64_t B,
                           const int64_t* values, const int32_t* lengths, const void* sums,
                           size_t sums_bytes, int64_t* offsets_out, float* out, int64_t* rows_out,
                           EmbArgs* a, bool* work) {
    const std::string f(fn);
    *work = false;
    if (!tables) return fail(REC_EINVAL, f + ": tables is NULL");
    if (T < 1) return fail(REC_EINVAL, f + ": T < 1");
    if (T > REC_MAX_TABLES) return fail(REC_EUNSUPPORTED, f + ": T > REC_MAX_TABLES");
    if (B < 0) return fail(REC_EINVAL, f + ": B < 0");
    if (!values || !lengths || !sums || !out)
        return fail(REC_EINVAL, f + ": values, lengths, sums and out are required");
    if (!aligned16(out)) return fail(REC_EINVAL, f + ": out not 16-byte aligned");
    if ((uintptr_t)sums & 7u) return fail(REC_EINVAL, f + ": sums not 8-byte aligned");
    if (sums_bytes < rec_kjt_sums_bytes(T, B))
        return fail(REC_EWORKSPACE, f + ": sums smaller than rec_kjt_sums_bytes(T, B)");
    memset(a, 0, sizeof(*a));
    for (int t = 0; t < T; ++t) {
        rec_status s = prep_table(tables[t], (f + ": table").c_str(), &a->tab[t]);
        if (s != REC_OK) return s;
    }
    const KjtLayout k = kjt_layout(T, B);
    a->values = values;
    a->lengths = lengths;
    a->offsets = nullptr;
    a->kjt_bs = (const int64_t*)sums;
    a->kjt_segp = (const int64_t*)((const char*)sums + k.off_segp);
    a->kjt_chp = (const int64_t*)((const char*)sums + k.off_chp);
    a->nK = k.nK;
    a->G = k.G;
    a->offsets_out = offsets_out;
    a->out = out;
    a->rows_out = rows_out;
    a->B = B;
    a->T = T;
    *work = B > 0;
    return REC_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

rec_status prep_towers(const char* fn, const rec_tower_mlp* mlp, int64_t B, const float* pooled,
                       int64_t pooled_ld, const float* att, float* deep_out, float* logit,
                       float* prob, TowerArgs* a, bool* work) {
    const std::string f(fn);
    *work = false;
    if (B < 0) return fail(REC_EINVAL, f + ": B < 0");
    if (!mlp) return fail(REC_EINVAL, f + ": tower mlp is NULL");
    if (mlp->dtype != REC_F32 && mlp->dtype != REC_BF16 && mlp->dtype != REC_BF16_PACKED)
        return fail(REC_EINVAL, f + ": tower dtype must be REC_F32, REC_BF16 or REC_BF16_PACKED");
    const bool packed = mlp->dtype == REC_BF16_PACKED;
    const void* arrays[] = {mlp->wd1, mlp->bd1, mlp->bd2, mlp->bd3, mlp->bf, mlp->wo,
                            packed ? mlp->wd1 : mlp->wd2, packed ? mlp->wd1 : mlp->wd3,
                            packed ? mlp->wd1 : mlp->wf};
    for (const void* p : arrays) {
        if (!p) return fail(REC_EINVAL, f + ": tower weights, biases and wo are required");
        if (!aligned16(p)) return fail(REC_EINVAL, f + ": tower arrays must be 16-byte aligned");
    }
    if (!pooled || !att || !logit) return fail(REC_EINVAL, f + ": pooled, att and logit are required");
    if (pooled_ld < 256 || (pooled_ld & 3))
        return fail(REC_EINVAL, f + ": pooled_ld must be >= 256 and a multiple of 4");
    if (!aligned16(pooled) || !aligned16(att) || (deep_out && !aligned16(deep_out)))
        return fail(REC_EINVAL, f + ": pooled, att and deep_out must be 16-byte aligned");
    if ((B + kTowerSamples - 1) / kTowerSamples > 2147483647LL)
        return fail(REC_EUNSUPPORTED, f + ": B too large for one launch");
    a->w[0] = mlp->wd1;
    a->w[1] = mlp->wd2;
    a->w[2] = mlp->wd3;
    a->w[3] = mlp->wf;
    a->b[0] = mlp->bd1;
    a->b[1] = mlp->bd2;
    a->b[2] = mlp->bd3;
    a->b[3] = mlp->bf;
    a->wo = mlp->wo;
    a->bo = mlp->bo;
    a->dtype = mlp->dtype;
    a->pooled = pooled;
    a->pooled_ld = pooled_ld;
    a->att = att;
    a->deep_out = deep_out;
    a->logit = logit;
    a->prob = prob;
    a->B = B;
    *work = B > 0;
    return REC_OK;
}

}  // namespace

bool rec::take_timing(int which, hipEvent_t* start, hipEvent_t* stop) {
    if (which < 0 || which >= REC_TIME_KINDS || !g_time[which][0]) return false;
    *start = g_time[which][0];
    *stop = g_time[which][1];
    g_time[which][0] = g_time[which][1] = nullptr;
    return true;
}

extern "C" {

rec_status rec_time_next_launch(int32_t kernel, void* start, void* stop) {
    if (kernel < 0 || kernel >= REC_TIME_KINDS) return fail(REC_EINVAL, "rec_time_next_launch: unknown kernel");
    if ((start == nullptr) != (stop == nullptr))
        return fail(REC_EINVAL, "rec_time_next_launch: give both events or neither");
    g_time[kernel][0] = (hipEvent_t)start;
    g_time[kernel][1] = (hipEvent_t)stop;
    return ok();
}

const char* rec_last_error(void) { return g_err.c_str(); }

int32_t rec_version(void) { return 100; }

int64_t rec_host_floor_mod(int64_t x, int64_t n) {
    if (n < 1) return -1;
    uint64_t m;
    int32_t s;
    floor_mod_prepare(n, &m, &s);
    return floor_mod_magic(x, n, m, s);
}

int64_t rec_host_hash_probe(const int64_t* keys, const uint8_t* digests, int64_t capacity,
                            int64_t key) {
    if (!keys || !digests || capacity < 1 || !aligned16(digests)) return -2;
    TabDev t;
    memset(&t, 0, sizeof(t));
    t.keys = keys;
    t.digests = digests;
    t.rows = capacity;
    t.kind = REC_HASH;
    return hash_probe(t, key);
}

int64_t rec_host_hash_home(int64_t x, int64_t capacity, uint8_t* digest) {
    const uint64_t h = mix64((uint64_t)x);
    if (digest) *digest = (uint8_t)hash_digest(h);
    return capacity >= 1 ? hash_home(h, capacity) : -1;
}

rec_status rec_lengths_to_offsets(const int32_t* lengths, int64_t n, int64_t* offsets, void* stream) {
    if (n < 0) return fail(REC_EINVAL, "rec_lengths_to_offsets: n < 0");
    if (!offsets) return fail(REC_EINVAL, "rec_lengths_to_offsets: offsets is NULL");
    if (n > 0 && !lengths) return fail(REC_EINVAL, "rec_lengths_to_offsets: lengths is NULL");
    if ((uintptr_t)offsets & 7u) return fail(REC_EINVAL, "rec_lengths_to_offsets: offsets not 8-byte aligned");
    return hip_status(launch_lengths_to_offsets(lengths, n, offsets, (hipStream_t)stream),
                      "rec_lengths_to_offsets");
}

rec_status rec_embbag_fwd(const rec_table* tables, int32_t T, int64_t B, const int64_t* values,
                          const int32_t* lengths, const int64_t* offsets, float* out,
                          int64_t* rows_out, void* stream) {
    if (!tables) return fail(REC_EINVAL, "rec_embbag_fwd: tables is NULL");
    if (T < 1) return fail(REC_EINVAL, "rec_embbag_fwd: T < 1");
    if (T > REC_MAX_TABLES) return fail(REC_EUNSUPPORTED, "rec_embbag_fwd: T > REC_MAX_TABLES");
    if (B < 0) return fail(REC_EINVAL, "rec_embbag_fwd: B < 0");
    if (!values || !lengths || !offsets || !out)
        return fail(REC_EINVAL, "rec_embbag_fwd: values, lengths, offsets and out are required");
    if (!aligned16(out)) return fail(REC_EINVAL, "rec_embbag_fwd: out not 16-byte aligned");
    EmbArgs a;
    memset(&a, 0, sizeof(a));
    for (int t = 0; t < T; ++t) {
        rec_status s = prep_table(tables[t], "rec_embbag_fwd: table", &a.tab[t]);
        if (s != REC_OK) return s;
    }
    if (B == 0) return ok();
    a.values = values;
    a.lengths = lengths;
    a.offsets = offsets;
    a.out = out;
    a.rows_out = rows_out;
    a.B = B;
    a.T = T;
    return hip_status(launch_embbag(a, (hipStream_t)stream), "rec_embbag_fwd");
}

size_t rec_kjt_sums_bytes(int32_t T, int64_t B) {
    if (T < 1 || T > REC_MAX_TABLES || B < 0) return 0;
    return kjt_layout(T, B).bytes;
}

rec_status rec_kjt_sums(const int32_t* lengths, int32_t T, int64_t B, void* sums,
                        size_t sums_bytes, void* stream) {
    if (T < 1) return fail(REC_EINVAL, "rec_kjt_sums: T < 1");
    if (T > REC_MAX_TABLES) return fail(REC_EUNSUPPORTED, "rec_kjt_sums: T > REC_MAX_TABLES");
    if (B < 0) return fail(REC_EINVAL, "rec_kjt_sums: B < 0");
    if (B > 0 && !lengths) return fail(REC_EINVAL, "rec_kjt_sums: lengths is NULL");
    if (!sums) return fail(REC_EINVAL, "rec_kjt_sums: sums is NULL");
    if ((uintptr_t)sums & 7u) return fail(REC_EINVAL, "rec_kjt_sums: sums not 8-byte aligned");
    if (sums_bytes < rec_kjt_sums_bytes(T, B))
        return fail(REC_EWORKSPACE, "rec_kjt_sums: sums smaller than rec_kjt_sums_bytes(T, B)");
    if (B == 0) return ok();
    return hip_status(launch_kjt_sums(lengths, T, B, sums, (hipStream_t)stream), "rec_kjt_sums");
}

rec_status rec_hash_lookup(const rec_table* table, const int64_t* keys, int64_t n,
                           int64_t* slot_out, float* rows_out, void* stream) {
    if (!table) return fail(REC_EINVAL, "rec_hash_lookup: table is NULL");
    if (table->kind != REC_HASH) return fail(REC_EINVAL, "rec_hash_lookup: table kind is not REC_HASH");
    if (n < 0) return fail(REC_EINVAL, "rec_hash_lookup: n < 0");
    if (!slot_out && !rows_out) return fail(REC_EINVAL, "rec_hash_lookup: no output requested");
    if (n > 0 && !keys) return fail(REC_EINVAL, "rec_hash_lookup: keys is NULL");
    if (rows_out && !aligned16(rows_out)) return fail(REC_EINVAL, "rec_hash_lookup: rows_out not 16-byte aligned");
    HashArgs a;
    memset(&a, 0, sizeof(a));
    rec_status s = prep_table(*table, "rec_hash_lookup: table", &a.tab);
    if (s != REC_OK) return s;
    if (n == 0) return ok();
    a.keys = keys;
    a.n = n;
    a.slot_out = slot_out;
    a.rows_out = rows_out;
    return hip_status(launch_hash_lookup(a, (hipStream_t)stream), "rec_hash_lookup");
}

size_t rec_hash_insert_workspace_bytes(int64_t n, int64_t capacity) {
    if (n < 0 || n > ((int64_t)1 << 30) || capacity < 1 || capacity > 2147483647LL) return 0;
    return align256(4 * (size_t)n) + 4 * (size_t)capacity;
}

rec_status rec_hash_insert(const rec_table* table, const int64_t* keys, const float* values,
                           int64_t n, int32_t score_mode, uint64_t step, int64_t* slot_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!table) return fail(REC_EINVAL, "rec_hash_insert: table is NULL");
    if (table->kind != REC_HASH) return fail(REC_EINVAL, "rec_hash_insert: table kind is not REC_HASH");
    if (n < 0) return fail(REC_EINVAL, "rec_hash_insert: n < 0");
    if (n > ((int64_t)1 << 30)) return fail(REC_EUNSUPPORTED, "rec_hash_insert: n above 2^30");
    if (score_mode != REC_SCORE_NONE && score_mode != REC_SCORE_STEP && score_mode != REC_SCORE_LFU)
        return fail(REC_EINVAL, "rec_hash_insert: unknown score_mode");
    if (score_mode != REC_SCORE_NONE && !table->scores)
        return fail(REC_EINVAL, "rec_hash_insert: this score_mode needs table scores");
    if (table->scores && ((uintptr_t)table->scores & 7))
        return fail(REC_EINVAL, "rec_hash_insert: scores not 8-byte aligned");
    if (n > 0 && (!keys || !values)) return fail(REC_EINVAL, "rec_hash_insert: keys or values is NULL");
    if (n > 0 && !aligned16(values)) return fail(REC_EINVAL, "rec_hash_insert: values not 16-byte aligned");
    HashArgs t;
    memset(&t, 0, sizeof(t));
    rec_status s = prep_table(*table, "rec_hash_insert: table", &t.tab);
    if (s != REC_OK) return s;
    if (n == 0) return ok();
    if (!workspace || workspace_bytes < rec_hash_insert_workspace_bytes(n, table->rows))
        return fail(REC_EWORKSPACE, "rec_hash_insert: workspace missing or smaller than rec_hash_insert_workspace_bytes(n, capacity)");
    if ((uintptr_t)workspace & 255u) return fail(REC_EINVAL, "rec_hash_insert: workspace not 256-byte aligned");
    HashInsArgs a;
    a.keys = const_cast<int64_t*>(table->keys);
    a.digests = const_cast<uint8_t*>(table->digests);
    a.scores = const_cast<uint64_t*>(table->scores);
    a.values = const_cast<float*>(table->values);
    a.capacity = table->rows;
    a.in_keys = keys;
    a.in_values = values;
    a.n = n;
    a.mode = score_mode;
    a.step = step;
    a.slot_out = slot_out;
    a.pair_slot = (int32_t*)workspace;
    a.winner = (int32_t*)((char*)workspace + align256(4 * (size_t)n));
    return hip_status(launch_hash_insert(a, (hipStream_t)stream), "rec_hash_insert");
}

size_t rec_hash_admit_workspace_bytes(int64_t n, int64_t capacity, int32_t score_mode) {
    if (n < 0 || n > ((int64_t)1 << 30) || capacity < 1 || capacity > 2147483647LL) return 0;
    return admit_layout(n, capacity, score_mode != REC_SCORE_NONE).bytes;
}

rec_status rec_hash_admit(const rec_table* table, int64_t max_keys, int64_t* counter_keys,
                          uint64_t* counter_counts, int64_t counter_capacity, const int64_t* keys,
                          const float* init_values, int64_t n, uint64_t threshold, int32_t score_mode,
                          uint64_t step, int64_t* slot_out, int64_t* counts_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
    const std::string f("rec_hash_admit");
    if (!table) return fail(REC_EINVAL, f + ": table is NULL");
    if (table->kind != REC_HASH) return fail(REC_EINVAL, f + ": table kind is not REC_HASH");
    HashArgs t;
    memset(&t, 0, sizeof(t));
    rec_status st = prep_table(*table, "rec_hash_admit: table", &t.tab);
    if (st != REC_OK) return st;
    if (n < 0) return fail(REC_EINVAL, f + ": n < 0");
    if (n > ((int64_t)1 << 30)) return fail(REC_EUNSUPPORTED, f + ": n above 2^30");
    if (score_mode != REC_SCORE_NONE && score_mode != REC_SCORE_STEP && score_mode != REC_SCORE_LFU)
        return fail(REC_EINVAL, f + ": unknown score_mode");
    if (score_mode != REC_SCORE_NONE && !table->scores)
        return fail(REC_EINVAL, f + ": this score_mode needs table scores");
    if (table->scores && ((uintptr_t)table->scores & 7)) return fail(REC_EINVAL, f + ": scores not 8-byte aligned");
    if (max_keys < 0 || max_keys > table->rows) return fail(REC_EINVAL, f + ": max_keys outside [0, capacity]");
    if (threshold < 1) return fail(REC_EINVAL, f + ": threshold must be >= 1");
    if (!counter_keys || !counter_counts || counter_capacity < 1)
        return fail(REC_EINVAL, f + ": a counter table (keys, counts, capacity >= 1) is required");
    if (((uintptr_t)counter_keys & 7) || ((uintptr_t)counter_counts & 7))
        return fail(REC_EINVAL, f + ": counter arrays not 8-byte aligned");
    if (n == 0) return ok();
    if (!keys || !init_values) return fail(REC_EINVAL, f + ": keys and init_values are required");
    if (!aligned16(init_values)) return fail(REC_EINVAL, f + ": init_values not 16-byte aligned");
    const AdmitLayout L = admit_layout(n, table->rows, score_mode != REC_SCORE_NONE);
    if (!workspace || workspace_bytes < L.bytes)
        return fail(REC_EWORKSPACE, f + ": workspace missing or smaller than rec_hash_admit_workspace_bytes");
    if ((uintptr_t)workspace & 255u) return fail(REC_EINVAL, f + ": workspace not 256-byte aligned");
    char* w = (char*)workspace;
    AdmitArgs a;
    memset(&a, 0, sizeof(a));
    a.tab = t.tab;
    a.keys = const_cast<int64_t*>(table->keys);
    a.digests = const_cast<uint8_t*>(table->digests);
    a.scores = const_cast<uint64_t*>(table->scores);
    a.values = const_cast<float*>(table->values);
    a.capacity = table->rows;
    a.max_keys = max_keys;
    a.ckeys = counter_keys;
    a.ccounts = counter_counts;
    a.ccap = counter_capacity;
    a.in_keys = keys;
    a.init_values = init_values;
    a.n = n;
    a.threshold = threshold;
    a.step = step;
    a.mode = score_mode;
    a.slot_out = slot_out;
    a.counts_out = counts_out;
    a.set_key = (int64_t*)(w + L.set_key);
    a.set_cnt = (uint32_t*)(w + L.set_cnt);
    a.set_first = (int32_t*)(w + L.set_first);
    a.nset = L.nset;
    a.flag = (int32_t*)(w + L.flag);
    a.rank = (int32_t*)(w + L.rank);
    a.total = (uint64_t*)(w + L.total);
    a.cslot = (int64_t*)(w + L.cslot);
    a.blk_cnt = (int32_t*)(w + L.blk_cnt);
    a.nbn = L.nbn;
    a.blk_stored = (int32_t*)(w + L.blk_stored);
    a.nbs = L.nbs;
    a.hdr = (int64_t*)(w + L.hdr);
    if (score_mode != REC_SCORE_NONE) {
        a.sel_hist = (uint32_t*)(w + L.sel_hist);
        a.sel_state = (int64_t*)(w + L.sel_state);
    }
    return hip_status(launch_hash_admit(a, (hipStream_t)stream), "rec_hash_admit");
}

rec_status rec_dlrm_interact(const float* z, int64_t B, int32_t F, int32_t d, float* out, void* stream) {
    if (B < 0) return fail(REC_EINVAL, "rec_dlrm_interact: B < 0");
    if (F < 1) return fail(REC_EINVAL, "rec_dlrm_interact: F < 1");
    if (d < 16 || d % 16 != 0) return fail(REC_EINVAL, "rec_dlrm_interact: d must be a positive multiple of 16");
    if (F > 256 || d > 512) return fail(REC_EUNSUPPORTED, "rec_dlrm_interact: F above 256 or d above 512");
    if ((int64_t)32 * ((F + 31) / 32) * dlrm_stride(d) > kDlrmMaxLdsFloats)
        return fail(REC_EUNSUPPORTED, "rec_dlrm_interact: F x d does not fit the 144 KiB LDS stage");
    if (B > 0 && (!z || !out)) return fail(REC_EINVAL, "rec_dlrm_interact: z or out is NULL");
    if (B > 0 && !aligned16(z)) return fail(REC_EINVAL, "rec_dlrm_interact: z not 16-byte aligned");
    if (B == 0) return ok();
    const int cus = num_cus();
    if (cus < 1) return fail(REC_EHIP, "rec_dlrm_interact: cannot query the device");
    return hip_status(launch_dlrm_interact(z, B, F, d, out, cus, (hipStream_t)stream), "rec_dlrm_interact");
}

rec_status rec_dlrm_fwd(const rec_dlrm_mlp* mlp, const rec_table* tables, const int32_t* modes,
                        int64_t B, const float* dense, const int64_t* values,
                        const int32_t* lengths, const int64_t* offsets, float* z, float* inter,
                        float* logit, float* prob, void* stream) {
    const std::string f("rec_dlrm_fwd");
    if (!mlp || !tables || !modes) return fail(REC_EINVAL, f + ": mlp, tables and modes are required");
    if (B < 0) return fail(REC_EINVAL, f + ": B < 0");
    const int32_t S = mlp->S, d = mlp->dim, nd = mlp->n_dense;
    if (S < 1 || S > kDlrmMaxTables) return fail(REC_EINVAL, f + ": S outside [1, 255]");
    if (d < 32 || d > 256 || d % 32) return fail(REC_EINVAL, f + ": dim must be a multiple of 32 in [32, 256]");
    if (nd < 1 || nd > kDlrmMaxDense) return fail(REC_EINVAL, f + ": n_dense outside [1, 128]");
    const bool wide = S > kDlrmMaxTablesFused || (S + 1) * d > kDlrmMaxZ;
    if (wide && (int64_t)32 * ((S + 1 + 31) / 32) * dlrm_stride(d) > kDlrmMaxLdsFloats)
        return fail(REC_EUNSUPPORTED, f + ": (S + 1) x dim does not fit the interaction's 144 KiB LDS stage");
    const void* arrays[] = {mlp->wb1, mlp->bb1, mlp->wb2, mlp->bb2, mlp->wt1, mlp->bt1, mlp->wt2,
                            mlp->bt2, mlp->wt3};
    for (const void* p : arrays) {
        if (!p) return fail(REC_EINVAL, f + ": mlp weights and biases are required");
        if (!aligned16(p)) return fail(REC_EINVAL, f + ": mlp arrays must be 16-byte aligned");
    }
    DlrmArgs a;
    memset(&a, 0, sizeof(a));
    std::vector<TabDev> tabs((size_t)S);
    std::vector<int32_t> md((size_t)S);
    for (int t = 0; t < S; ++t) {
        const rec_table& tb = tables[t];
        if (tb.kind != REC_DIRECT) return fail(REC_EINVAL, f + ": tables must be REC_DIRECT");
        if (tb.dim != d) return fail(REC_EINVAL, f + ": a table's dim differs from mlp->dim");
        if (tb.rows < 1) return fail(REC_EINVAL, f + ": rows must be >= 1");
        if (!tb.values || !aligned16(tb.values)) return fail(REC_EINVAL, f + ": table values NULL or misaligned");
        if (modes[t] != REC_POOL_SUM && modes[t] != REC_POOL_MEAN) return fail(REC_EINVAL, f + ": unknown mode");
        memset(&tabs[t], 0, sizeof(TabDev));
        tabs[t].values = tb.values;
        tabs[t].rows = tb.rows;
        tabs[t].kind = REC_DIRECT;
        floor_mod_prepare(tb.rows, &tabs[t].magic, &tabs[t].shift);
        md[t] = modes[t];
        if (t < 32) {
            a.tab[t] = tabs[t];
            a.mode[t] = md[t];
        }
    }
    if (B == 0) return ok();
    if (!dense || !values || !lengths || !offsets || !z || !logit)
        return fail(REC_EINVAL, f + ": dense, values, lengths, offsets, z and logit are required");
    if (!aligned16(z)) return fail(REC_EINVAL, f + ": z not 16-byte aligned");
    if (wide && !inter) return fail(REC_EINVAL, f + ": inter is required for more than 31 tables or (S + 1) * dim above 1024");
    a.B = B;
    a.S = S;
    a.dim = d;
    a.n_dense = nd;
    a.dense = dense;
    a.values = values;
    a.lengths = lengths;
    a.offsets = offsets;
    a.wb1 = mlp->wb1;
    a.bb1 = mlp->bb1;
    a.wb2 = mlp->wb2;
    a.bb2 = mlp->bb2;
    a.wt1 = mlp->wt1;
    a.bt1 = mlp->bt1;
    a.wt2 = mlp->wt2;
    a.bt2 = mlp->bt2;
    a.wt3 = mlp->wt3;
    a.bt3 = mlp->bt3;
    a.z = z;
    a.inter = inter;
    a.logit = logit;
    a.prob = prob;
    if (wide) {
        const int cus = num_cus();
        if (cus < 1) return fail(REC_EHIP, f + ": cannot query the device");
        return hip_status(launch_dlrm_fwd_wide(a, tabs.data(), md.data(), cus, (hipStream_t)stream), "rec_dlrm_fwd");
    }
    return hip_status(launch_dlrm_fwd(a, (hipStream_t)stream), "rec_dlrm_fwd");
}

rec_status rec_hash_clear(const rec_table* table, void* stream) {
    if (!table) return fail(REC_EINVAL, "rec_hash_clear: table is NULL");
    if (table->kind != REC_HASH) return fail(REC_EINVAL, "rec_hash_clear: table kind is not REC_HASH");
    if (table->scores && ((uintptr_t)table->scores & 7))
        return fail(REC_EINVAL, "rec_hash_clear: scores not 8-byte aligned");
    HashArgs t;
    memset(&t, 0, sizeof(t));
    rec_status s = prep_table(*table, "rec_hash_clear: table", &t.tab);
    if (s != REC_OK) return s;
    return hip_status(launch_hash_clear(const_cast<int64_t*>(table->keys), const_cast<uint8_t*>(table->digests),
                                        const_cast<uint64_t*>(table->scores), table->rows, (hipStream_t)stream),
                      "rec_hash_clear");
}

rec_status rec_din_pack_mlp(const rec_din_mlp* mlp, void* packed, size_t packed_bytes, void* stream) {
    if (!mlp) return fail(REC_EINVAL, "rec_din_pack_mlp: mlp is NULL");
    if (mlp->dtype != REC_BF16) return fail(REC_EINVAL, "rec_din_pack_mlp: dtype must be REC_BF16");
    if (!mlp->w1 || !mlp->w2) return fail(REC_EINVAL, "rec_din_pack_mlp: w1 and w2 are required");
    if (!packed) return fail(REC_EINVAL, "rec_din_pack_mlp: packed is NULL");
    if (!aligned16(mlp->w1) || !aligned16(mlp->w2) || !aligned16(packed))
        return fail(REC_EINVAL, "rec_din_pack_mlp: pointers must be 16-byte aligned");
    if (packed_bytes < REC_DIN_PACKED_BYTES)
        return fail(REC_EWORKSPACE, "rec_din_pack_mlp: packed smaller than REC_DIN_PACKED_BYTES");
    return hip_status(launch_din_pack(mlp->w1, mlp->w2, packed, (hipStream_t)stream), "rec_din_pack_mlp");
}

size_t rec_din_plan_bytes(int64_t B, int32_t max_len) {
    if (B < 0 || max_len < 1 || max_len > REC_MAX_SEQ_LEN || B > REC_MAX_B) return 0;
    return plan_layout(B, max_len).bytes;
}

rec_status rec_din_plan(const rec_table* seq_tables, const int64_t* seq_values,
                        int64_t seq_stride, const int64_t* seq_offsets,
                        const int32_t* seq_lengths, int64_t B, int32_t max_len,
                        int32_t range_positions, int64_t* seq_offsets_out, int64_t* rows_out,
                        void* plan, size_t plan_bytes, void* stream) {
    PlanArgs a;
    bool work;
    rec_status s = prep_plan("rec_din_plan", seq_tables, seq_values, seq_stride, seq_offsets,
                             seq_lengths, B, max_len, range_positions, seq_offsets_out, rows_out,
                             plan, plan_bytes, &a, &work);
    if (s != REC_OK) return s;
    if (!work) return ok();
    const int cus = num_cus();
    if (cus < 1) return fail(REC_EHIP, "rec_din_plan: cannot query the device");
    a.waves = din_waves(cus);
    return hip_status(launch_din_plan(a, (hipStream_t)stream), "rec_din_plan");
}

rec_status rec_din_attn_fwd_plan(const rec_table* seq_tables, const void* plan, size_t plan_bytes,
                                 int64_t B, int32_t max_len, const float* query, int64_t query_ld,
                                 const int32_t* query_col, const rec_din_mlp* mlp, float* out,
                                 float* scores_out, float* weights_out, void* stream) {
    DinArgs a;
    bool work;
    rec_status s = prep_attn("rec_din_attn_fwd_plan", seq_tables, plan, plan_bytes, B, max_len, query,
                             query_ld, query_col, mlp, out, scores_out, weights_out, &a, &work);
    if (s != REC_OK) return s;
    if (!work) return ok();
    const int cus = num_cus();
    if (cus < 1) return fail(REC_EHIP, "rec_din_attn_fwd_plan: cannot query the device");
    a.waves = din_waves(cus);
    return hip_status(launch_din(a, (hipStream_t)stream), "rec_din_attn_fwd_plan");
}

size_t rec_din_attn_workspace_bytes(int64_t B, int32_t max_len) { return rec_din_plan_bytes(B, max_len); }

rec_status rec_din_attn_fwd(const rec_table* seq_tables, const int64_t* seq_values, int64_t seq_stride,
                            const int64_t* seq_offsets, const int32_t* seq_lengths, int32_t max_len,
                            int64_t B, const float* query, int64_t query_ld, const int32_t* query_col,
                            const rec_din_mlp* mlp, float* out, float* scores_out, float* weights_out,
                            int64_t* rows_out, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "rec_din_attn_fwd";
    PlanArgs p;
    DinArgs d;
    bool wp, wd;
    rec_status s = prep_plan(fn, seq_tables, seq_values, seq_stride, seq_offsets, seq_lengths, B,
                             max_len, 0, nullptr, rows_out, workspace, workspace_bytes, &p, &wp,
                             "workspace", "rec_din_attn_workspace_bytes");
    if (s != REC_OK) return s;
    s = prep_attn(fn, seq_tables, workspace, workspace_bytes, B, max_len, query, query_ld, query_col,
                  mlp, out, scores_out, weights_out, &d, &wd, "workspace", "rec_din_attn_workspace_bytes");
    if (s != REC_OK) return s;
    if (!wp || !wd) return ok();
    const int cus = num_cus();
    if (cus < 1) return fail(REC_EHIP, "rec_din_attn_fwd: cannot query the device");
    p.waves = d.waves = din_waves(cus);
    hipError_t h = launch_din_plan(p, (hipStream_t)stream);
    if (h == hipSuccess) h = launch_din(d, (hipStream_t)stream);
    return hip_status(h, fn);
}

rec_status rec_embbag_fwd_kjt(const rec_table* tables, int32_t T, int64_t B,
                              const int64_t* values, const int32_t* lengths, const void* sums,
                              size_t sums_bytes, int64_t* offsets_out, float* out,
                              int64_t* rows_out, void* stream) {
    EmbArgs a;
    bool work;
    rec_status s = prep_embbag_kjt("rec_embbag_fwd_kjt", tables, T, B, values, lengths, sums,
                                   sums_bytes, offsets_out, out, rows_out, &a, &work);
    if (s != REC_OK) return s;
    if (!work) return ok();
    return hip_status(launch_embbag(a, (hipStream_t)stream), "rec_embbag_fwd_kjt");
}

size_t rec_sparse_din_fwd_workspace_bytes(int32_t T, int64_t B, int32_t max_len) {
    const size_t k = rec_kjt_sums_bytes(T, B), p = rec_din_plan_bytes(B, max_len);
    if ((k == 0 && B > 0) || p == 0) return 0;
    return align256(k) + p;
}

}  // extern "C"

namespace {

// rec_sparse_din_fwd's checks and kernel arguments for a given workspace;
// *work is false when there is nothing to launch.  No HIP call.
rec_status prep_whole(const char* fn, const rec_fwd_args* x, char* ws, size_t wsb, EmbArgs* e,
                      PlanArgs* p, DinArgs* d, bool* work) {
    *work = false;
    const size_t need = rec_sparse_din_fwd_workspace_bytes(x->T, x->B, x->max_len);
    if (need == 0 && (x->T < 1 || x->T > REC_MAX_TABLES || x->B < 0))
        return fail(REC_EINVAL, std::string(fn) + ": T or B out of range");
    if (wsb < need)
        return fail(REC_EWORKSPACE, std::string(fn) + ": workspace smaller than rec_sparse_din_fwd_workspace_bytes");
    const size_t kb = align256(rec_kjt_sums_bytes(x->T, x->B));
    bool we, wp, wd;
    rec_status s = prep_embbag_kjt(fn, x->tables, x->T, x->B, x->values, x->lengths, ws, kb,
                                   x->offsets_out, x->pooled, x->rows_out, e, &we);
    if (s != REC_OK) return s;
    s = prep_plan(fn, x->seq_tables, x->seq_values, x->seq_stride, x->seq_offsets, x->seq_lengths,
                  x->B, x->max_len, x->range_positions, x->seq_offsets_out, x->seq_rows_out,
                  ws + kb, wsb - kb, p, &wp);
    if (s != REC_OK) return s;
    s = prep_attn(fn, x->seq_tables, ws + kb, wsb - kb, x->B, x->max_len, x->pooled,
                  (int64_t)x->T * 16, x->query_col, x->mlp, x->att, x->scores_out, x->weights_out,
                  d, &wd);
    if (s != REC_OK) return s;
    *work = we && wp && wd;
    return REC_OK;
}

rec_status launch_whole(const char* fn, EmbArgs& e, PlanArgs& p, DinArgs& d, void* stream) {
    const int cus = num_cus();
    if (cus < 1) return fail(REC_EHIP, std::string(fn) + ": cannot query the device");
    p.waves = d.waves = din_waves(cus);
    hipError_t h = launch_fwd_front(p, e, (hipStream_t)stream);
    if (h == hipSuccess) h = launch_din(d, (hipStream_t)stream);
    return hip_status(h, fn);
}

}  // namespace

extern "C" {

rec_status rec_sparse_din_fwd(const rec_fwd_args* x, void* stream) {
    const char* fn = "rec_sparse_din_fwd";
    if (!x) return fail(REC_EINVAL, "rec_sparse_din_fwd: args is NULL");
    if (!x->workspace) return fail(REC_EINVAL, "rec_sparse_din_fwd: workspace is NULL");
    if (!aligned16(x->workspace)) return fail(REC_EINVAL, "rec_sparse_din_fwd: workspace not 16-byte aligned");
    EmbArgs e;
    PlanArgs p;
    DinArgs d;
    bool work;
    rec_status s = prep_whole(fn, x, (char*)x->workspace, x->workspace_bytes, &e, &p, &d, &work);
    if (s != REC_OK) return s;
    if (!work) return ok();
    return launch_whole(fn, e, p, d, stream);
}

rec_status rec_tower_pack_mlp(const rec_tower_mlp* mlp, void* packed, size_t packed_bytes,
                              void* stream) {
    const char* fn = "rec_tower_pack_mlp";
    if (!mlp) return fail(REC_EINVAL, std::string(fn) + ": mlp is NULL");
    if (mlp->dtype != REC_BF16) return fail(REC_EINVAL, std::string(fn) + ": dtype must be REC_BF16");
    const void* w[4] = {mlp->wd1, mlp->wd2, mlp->wd3, mlp->wf};
    for (const void* p : w)
        if (!p) return fail(REC_EINVAL, std::string(fn) + ": wd1, wd2, wd3 and wf are required");
    if (!packed) return fail(REC_EINVAL, std::string(fn) + ": packed is NULL");
    for (const void* p : w)
        if (!aligned16(p)) return fail(REC_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
    if (!aligned16(packed)) return fail(REC_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
    if (packed_bytes < REC_TOWER_PACKED_BYTES)
        return fail(REC_EWORKSPACE, std::string(fn) + ": packed smaller than REC_TOWER_PACKED_BYTES");
    return hip_status(launch_tower_pack(w, packed, (hipStream_t)stream), fn);
}

rec_status rec_towers_fwd(const rec_tower_mlp* mlp, int64_t B, const float* pooled,
                          int64_t pooled_ld, const float* att, float* deep_out, float* logit,
                          float* prob, void* stream) {
    TowerArgs a;
    bool work;
    rec_status s = prep_towers("rec_towers_fwd", mlp, B, pooled, pooled_ld, att, deep_out, logit,
                               prob, &a, &work);
    if (s != REC_OK) return s;
    if (!work) return ok();
    return hip_status(launch_towers(a, (hipStream_t)stream), "rec_towers_fwd");
}

}  // extern "C"

namespace {

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Regions of rec_embbag_adagrad's workspace, in order: keys and sources in,
// their sort partners, head and tail pieces, the sort's per-tile digit counts
// and digit totals.
struct BwdLayout {
    size_t keys_in, src_in, keys_out, src_out, hpart, tpart, hist, tot, bytes;
};

bool bwd_layout(int64_t n, BwdLayout* L) {
    const size_t nb = round256((size_t)n * 4);
    const size_t nch = (size_t)((n + 15) / 16);
    const size_t pb = round256(nch * 16 * 4);
    L->keys_in = 0;
    L->src_in = L->keys_in + nb;
    L->keys_out = L->src_in + nb;
    L->src_out = L->keys_out + nb;
    L->hpart = L->src_out + nb;
    L->tpart = L->hpart + pb;
    L->hist = L->tpart + pb;
    L->tot = L->hist + round256((size_t)bwd_sort_tiles(n) * 256 * 4);
    L->bytes = L->tot + round256(256 * 4);
    return true;
}

}  // namespace

size_t rec_embbag_adagrad_workspace_bytes(int32_t T, int64_t B, int64_t nnz, int64_t P) {
    if (T < 1 || T > REC_MAX_TABLES || B < 0 || nnz < 0 || P < 0) return 0;
    const int64_t n = nnz + 3 * P;
    if (n >= ((int64_t)1 << 31) || B * T + 3 * P >= ((int64_t)1 << 31)) return 0;
    if (n == 0) return 0;
    BwdLayout L;
    if (!bwd_layout(n, &L)) return 0;
    return L.bytes;
}

rec_status rec_embbag_adagrad(const rec_adagrad_table* tables, int32_t T, int64_t B,
                              const int64_t* values, const int32_t* lengths,
                              const int64_t* offsets, int64_t nnz, const float* grad_pooled,
                              const int32_t* seq_table, const int64_t* seq_values,
                              int64_t seq_stride, int64_t P, const float* grad_seq, float lr,
                              float eps, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "rec_embbag_adagrad";
    const std::string f(fn);
    if (!tables) return fail(REC_EINVAL, f + ": tables is NULL");
    if (T < 1) return fail(REC_EINVAL, f + ": T < 1");
    if (T > REC_MAX_TABLES) return fail(REC_EUNSUPPORTED, f + ": T > REC_MAX_TABLES");
    if (B < 0 || nnz < 0 || P < 0) return fail(REC_EINVAL, f + ": B, nnz and P must be >= 0");
    const int64_t n = nnz + 3 * P;
    if (n >= ((int64_t)1 << 31) || B * T + 3 * P >= ((int64_t)1 << 31))
        return fail(REC_EUNSUPPORTED, f + ": nnz + 3P or B*T + 3P at 2^31 or more");
    BwdTab tabs[REC_MAX_TABLES];
    uint64_t total = 0;
    for (int t = 0; t < T; ++t) {
        const rec_adagrad_table& a = tables[t];
        if (!a.weights || !a.accum) return fail(REC_EINVAL, f + ": table weights or accum is NULL");
        if (!aligned16(a.weights) || !aligned16(a.accum))
            return fail(REC_EINVAL, f + ": table weights and accum must be 16-byte aligned");
        rec_table rt;
        memset(&rt, 0, sizeof(rt));
        rt.kind = a.kind;
        rt.dim = REC_DIM;
        rt.rows = a.rows;
        rt.values = a.weights;
        rt.keys = a.keys;
        rt.digests = a.digests;
        rec_status st = prep_table(rt, (f + ": table").c_str(), &tabs[t].tab);
        if (st != REC_OK) return st;
        tabs[t].weights = a.weights;
        tabs[t].accum = a.accum;
        tabs[t].rows = a.rows;
        tabs[t].base = (uint32_t)total;
        tabs[t].pad_ = 0;
        total += (uint64_t)a.rows;
        if (total >= ((uint64_t)1 << 32) - 1)
            return fail(REC_EUNSUPPORTED, f + ": table rows sum to 2^32 - 1 or more");
    }
    if (nnz > 0 && (!values || !lengths || !offsets || !grad_pooled))
        return fail(REC_EINVAL, f + ": values, lengths, offsets and grad_pooled are required when nnz > 0");
    if (nnz > 0 && B == 0) return fail(REC_EINVAL, f + ": nnz > 0 with B == 0");
    if (grad_pooled && !aligned16(grad_pooled)) return fail(REC_EINVAL, f + ": grad_pooled not 16-byte aligned");
    BwdArgs a;
    memset(&a, 0, sizeof(a));
    if (P > 0) {
        if (!seq_table || !seq_values || !grad_seq)
            return fail(REC_EINVAL, f + ": seq_table, seq_values and grad_seq are required when P > 0");
        if (seq_stride < P) return fail(REC_EINVAL, f + ": seq_stride < P");
        if (!aligned16(grad_seq)) return fail(REC_EINVAL, f + ": grad_seq not 16-byte aligned");
        for (int k = 0; k < 3; ++k) {
            if (seq_table[k] < 0 || seq_table[k] >= T) return fail(REC_EINVAL, f + ": seq_table entry outside [0, T)");
            a.seq_table[k] = seq_table[k];
        }
    }
    if (n == 0) return ok();
    BwdLayout L;
    bwd_layout(n, &L);
    if (!workspace || workspace_bytes < L.bytes) return fail(REC_EWORKSPACE, f + ": workspace missing or too small");
    if ((uintptr_t)workspace & 255u) return fail(REC_EINVAL, f + ": workspace not 256-byte aligned");
    char* w = (char*)workspace;
    a.values = values;
    a.lengths = lengths;
    a.offsets = offsets;
    a.grad_pooled = grad_pooled;
    a.seq_values = seq_values;
    a.grad_seq = grad_seq;
    a.seq_stride = seq_stride;
    a.B = B;
    a.nnz = nnz;
    a.P = P;
    a.n = n;
    a.T = T;
    a.total_rows = (uint32_t)total;
    a.lr = lr;
    a.eps = eps;
    a.keys_in = (uint32_t*)(w + L.keys_in);
    a.src_in = (uint32_t*)(w + L.src_in);
    a.hpart = (float*)(w + L.hpart);
    a.tpart = (float*)(w + L.tpart);
    // the sort covers every key up to `total` itself (a hash miss's key)
    int bits = 1;
    while (bits < 32 && ((uint64_t)1 << bits) <= total) ++bits;
    return hip_status(launch_embbag_adagrad(a, tabs, (uint32_t*)(w + L.keys_out), (uint32_t*)(w + L.src_out),
                                            (uint32_t*)(w + L.hist), (uint32_t*)(w + L.tot), bits,
                                            (hipStream_t)stream),
                      fn);
}

namespace {

struct DinBwdLayout {
    size_t w1t, w2t, map, S, X, H1, H2, E, PW, DE, DZ1, DZ2, GQP, part, bytes;
};

// The transposed weights and the per-position rows always; the split sums of
// the weight gradients only when they are requested.
DinBwdLayout din_bwd_layout(int64_t stride, bool weight_grads) {
    DinBwdLayout L;
    const size_t n = (size_t)stride;
    L.w1t = 0;
    L.w2t = L.w1t + round256(192 * 256 * 4);
    L.map = L.w2t + round256(256 * 64 * 4);
    L.S = L.map + round256(n * 4);
    L.X = L.S + round256(n * 48 * 4);
    L.H1 = L.X + round256(n * 193 * 4);
    L.H2 = L.H1 + round256(n * 257 * 4);
    L.E = L.H2 + round256(n * 65 * 4);
    L.PW = L.E + round256(n * 4);
    L.DE = L.PW + round256(n * 4);
    L.DZ1 = L.DE + round256(n * 4);
    L.DZ2 = L.DZ1 + round256(n * 256 * 4);
    L.GQP = L.DZ2 + round256(n * 64 * 4);
    L.part = L.GQP + round256(n * 48 * 4);
    L.bytes = L.part + (weight_grads ? round256((size_t)din_bwd_splits() * (size_t)din_bwd_part_stride() * 4) : 0);
    return L;
}

}  // namespace

size_t rec_din_attn_bwd_workspace_bytes(int64_t seq_stride, int32_t weight_grads) {
    if (seq_stride < 0) return 0;
    return din_bwd_layout(seq_stride, weight_grads != 0).bytes;
}

rec_status rec_din_attn_bwd(const rec_table* seq_tables, const int64_t* seq_values,
                            int64_t seq_stride, const int64_t* seq_offsets,
                            const int32_t* seq_lengths, int32_t max_len, int64_t B,
                            const float* query, int64_t query_ld, const int32_t* query_col,
                            const rec_din_mlp* mlp, const float* grad_att, float* grad_query,
                            float* grad_seq, float* dw1, float* db1, float* dw2, float* db2,
                            float* dw3, float* db3, void* workspace, size_t workspace_bytes,
                            void* stream) {
    const std::string f("rec_din_attn_bwd");
    if (B < 0) return fail(REC_EINVAL, f + ": B < 0");
    if (max_len < 1 || max_len > REC_MAX_SEQ_LEN) return fail(REC_EINVAL, f + ": max_len outside [1, REC_MAX_SEQ_LEN]");
    if (seq_stride < 0) return fail(REC_EINVAL, f + ": seq_stride < 0");
    if (!seq_tables || !mlp || !query_col) return fail(REC_EINVAL, f + ": seq_tables, mlp and query_col are required");
    if (mlp->dtype == REC_BF16_PACKED) return fail(REC_EUNSUPPORTED, f + ": packed MLP weights are not supported");
    if (mlp->dtype != REC_F32 && mlp->dtype != REC_BF16) return fail(REC_EINVAL, f + ": unknown dtype");
    const int nw = (dw1 != nullptr) + (db1 != nullptr) + (dw2 != nullptr) + (db2 != nullptr) +
                   (dw3 != nullptr) + (db3 != nullptr);
    if (nw != 0 && nw != 6) return fail(REC_EINVAL, f + ": give all six weight-gradient outputs or none");
    DinBwdArgs a;
    memset(&a, 0, sizeof(a));
    for (int k = 0; k < 3; ++k) {
        rec_status st = prep_table(seq_tables[k], (f + ": seq table").c_str(), &a.tabs[k]);
        if (st != REC_OK) return st;
        if (query_col[k] < 0 || query_col[k] + 16 > query_ld)
            return fail(REC_EINVAL, f + ": query_col outside the query row");
        a.qcol[k] = query_col[k];
    }
    if (B > 0 && (!seq_values || !seq_offsets || !seq_lengths || !query || !grad_att || !grad_query ||
                  !mlp->w1 || !mlp->w2 || !mlp->w3))
        return fail(REC_EINVAL, f + ": a required pointer is NULL");
    if (grad_seq && !aligned16(grad_seq)) return fail(REC_EINVAL, f + ": grad_seq not 16-byte aligned");
    const size_t need = rec_din_attn_bwd_workspace_bytes(seq_stride, nw == 6);
    if (!workspace || workspace_bytes < need) return fail(REC_EWORKSPACE, f + ": workspace missing or too small");
    if ((uintptr_t)workspace & 255u) return fail(REC_EINVAL, f + ": workspace not 256-byte aligned");
    if (B == 0) return ok();
    a.seq_values = seq_values;
    a.seq_stride = seq_stride;
    a.seq_offsets = seq_offsets;
    a.seq_lengths = seq_lengths;
    a.max_len = max_len;
    a.bf16 = mlp->dtype == REC_BF16;
    a.B = B;
    a.query = query;
    a.query_ld = query_ld;
    a.b3 = mlp->b3;
    a.w1 = mlp->w1;
    a.b1 = mlp->b1;
    a.w2 = mlp->w2;
    a.b2 = mlp->b2;
    a.w3 = mlp->w3;
    a.gatt = grad_att;
    a.gq = grad_query;
    a.gs = grad_seq;
    const DinBwdLayout L = din_bwd_layout(seq_stride, nw == 6);
    char* w = (char*)workspace;
    a.w1t = (float*)(w + L.w1t);
    a.w2t = (float*)(w + L.w2t);
    a.map = (int32_t*)(w + L.map);
    a.S = (float*)(w + L.S);
    a.X = (float*)(w + L.X);
    a.H1 = (float*)(w + L.H1);
    a.H2 = (float*)(w + L.H2);
    a.E = (float*)(w + L.E);
    a.PW = (float*)(w + L.PW);
    a.DE = (float*)(w + L.DE);
    a.DZ1 = (float*)(w + L.DZ1);
    a.DZ2 = (float*)(w + L.DZ2);
    a.GQP = (float*)(w + L.GQP);
    a.wgrad = nw == 6;
    if (nw == 6) {
        a.part = (float*)(w + L.part);
        a.part_stride = din_bwd_part_stride();
        a.dw1 = dw1;
        a.db1 = db1;
        a.dw2 = dw2;
        a.db2 = db2;
        a.dw3 = dw3;
        a.db3 = db3;
    }
    return hip_status(launch_din_bwd(a, (hipStream_t)stream), "rec_din_attn_bwd");
}

// ---------------------------------------------------------------------------
// rec_sparse_din_fwd_noalloc: the whole forward with its workspace (the KJT
// sums and the plan) in a static device array instead of a caller's buffer.
// Each device holds its own copy of the array, from the library's load until
// the process ends; the host side takes the array's device address once per
// device (hipGetSymbolAddress, under a lock) and passes that address to the
// kernels, never the array's name.
static __device__ __align__(256) unsigned char scratch[REC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

rec_status scratch_of_current_device(const char* fn, void** out) {
    int dev = -1;
    hipError_t h = hipGetDevice(&dev);
    if (h != hipSuccess) return hip_status(h, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(REC_EUNSUPPORTED, std::string(fn) + ": device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        h = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (h != hipSuccess) return hip_status(h, fn);
        if (!p) return fail(REC_EHIP, std::string(fn) + ": no device address for the static scratch");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return REC_OK;
}

}  // namespace

rec_status rec_sparse_din_fwd_noalloc(const rec_fwd_args* x, void* stream) {
    const char* fn = "rec_sparse_din_fwd_noalloc";
    if (!x) return fail(REC_EINVAL, "rec_sparse_din_fwd_noalloc: args is NULL");
    const size_t need = rec_sparse_din_fwd_workspace_bytes(x->T, x->B, x->max_len);
    if (need > REC_NOALLOC_SCRATCH_BYTES)
        return fail(REC_EWORKSPACE, "rec_sparse_din_fwd_noalloc: this batch needs " + std::to_string(need) +
                                        " bytes of workspace; the static scratch holds REC_NOALLOC_SCRATCH_BYTES = " +
                                        std::to_string((size_t)REC_NOALLOC_SCRATCH_BYTES));
    EmbArgs e;
    PlanArgs p;
    DinArgs d;
    bool work;
    // every check first, against a stand-in address with the scratch's
    // alignment (nothing is dereferenced on the host), so a rejected call
    // touches no device
    char* const stand_in = (char*)(uintptr_t)256;
    rec_status s = prep_whole(fn, x, stand_in, REC_NOALLOC_SCRATCH_BYTES, &e, &p, &d, &work);
    if (s != REC_OK) return s;
    if (!work) return ok();
    void* ws = nullptr;
    s = scratch_of_current_device(fn, &ws);
    if (s != REC_OK) return s;
    s = prep_whole(fn, x, (char*)ws, REC_NOALLOC_SCRATCH_BYTES, &e, &p, &d, &work);
    if (s != REC_OK) return s;
    return launch_whole(fn, e, p, d, stream);
}
