// Per-(b, KV head) selection: top-K of the block scores, then the residency
// diff with a capped fetch and LRU slot assignment.
//
// Top-K -- OasisKV explainer page (explanatory diagram, Fig. 7): predict the
// K blocks of the next step from the scores; K = budget_tokens / block_size.
// Order: higher score first, equal scores by lower block id; -0 equals +0.
// One workgroup per unit.  Scores become order-preserving 32-bit keys held in
// registers (each thread owns a contiguous id range).  The K'-th largest key
// (K' = min(K, NB)) is built bit by bit below the common prefix of the
// largest and smallest key with block-wide counts, stopping as soon as
// exactly K' keys reach the candidate.  Equal keys at the threshold are taken
// in id order through a block scan, which makes the choice among ties
// deterministic.  The K' winners are placed by rank counting, an exact sort
// for distinct (key, id) pairs.
//
// Select -- the explanatory diagram compares the predicted blocks with the
// blocks already on the GPU and transfers only the missing ones, capping the
// per-step transfer; the capped-eviction glossary entry bounds the blocks
// newly loaded in one step; Table 2 sets that cap by a fetch ratio and evicts
// LRU; Fig. 9 keeps, per KV head, a table from each GPU block (slot) to its
// CPU block.  Integer work only, per unit:
//   hits   = selected blocks held by a slot, in top-K order;
//   misses = selected blocks not held, in top-K order; the first
//            n = min(cap, |misses|) are fetched;
//   slots  = empty slots in ascending index, then slots of held blocks that
//            are not selected, least recently used first, ties to the lower
//            block id;
//   every hit and every fetched block gets last_used = t.
// The attended list is the hits followed by the fetched blocks; under the
// attend-all reading (every block held after the step) the held blocks that
// were neither selected nor evicted come between them, in slot order.  One
// wave does it: ordered compactions use ballots; victims are ranked by counting
// smaller (last_used, block) keys, exact because held block ids are distinct.
//
// The fused kernel runs both for a unit in one workgroup: the slot tables are
// copied into LDS while the top-K runs, and the winners go straight from LDS
// into the select.
#include "kernels.h"
#include "score_tile.h"

namespace oasis {

constexpr int kTopkMaxK = 1024;

__device__ __forceinline__ uint32_t order_key(float f, bool &bad) {
    uint32_t b = __float_as_uint(f);
    if (!isfinite(f)) {
        bad = true;
        return 0u;
    }
    if (b == 0x80000000u) b = 0u;  // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Lane (lane ^ J)'s value.  J < 16 stays inside a 16-lane row and goes
// through DPP: quad_perm [1,0,3,2] and [2,3,0,1] for 1 and 2, row_shl:4 /
// row_shr:4 chosen by lane bit 2 for 4, row_ror:8 for 8.  J = 16, 32 use a
// cross-lane shuffle.
template <int J> __device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
    const int x = (int)v;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    } else if constexpr (J == 4) {
        const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);  // lane + 4
        const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // lane - 4
        return (uint32_t)((threadIdx.x & 4) ? dn : up);
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
    } else {
        return (uint32_t)__shfl_xor(x, J, 64);
    }
}
template <int J> __device__ __forceinline__ unsigned long long lane_xor_u64(unsigned long long v) {
    const uint32_t lo = lane_xor_u32<J>((uint32_t)v), hi = lane_xor_u32<J>((uint32_t)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

// Inclusive suffix sum over the lanes of a wave (lane l: sum of lanes >= l):
// row_shl 1, 2, 4, 8 inside each 16-lane row, then the totals of the rows
// above, read from their first lanes.
__device__ __forceinline__ uint32_t wave_suffix_sum_u32(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x101, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x102, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x108, 0xF, 0xF, false);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t t3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row < 1 ? t1 : 0u) + (row < 2 ? t2 : 0u) + (row < 3 ? t3 : 0u);
}

template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sh[w];
    return base + x - v;
}

// Top-K of one unit's scores s[0..NB) into out[0..K) (and out2, out_lds when
// not null), -1 padded.  Called by every thread of an NT-thread workgroup.
//
// Radix select on the order keys: below the common high bits of the largest
// and smallest key, 8 bits per pass, an LDS histogram of the keys still in
// play picks the digit holding the K'-th largest key; it stops as soon as a
// digit's bin holds exactly the keys still needed.  If the bits run out first
// the bin is one key value tau and the lowest ids among the keys equal to tau
// fill the rest.
// One thread's share of a unit's scores: C = ceil(NB / NT) consecutive block
// ids starting at tid * C, as order keys.  Loaded first so that the loads
// overlap whatever the caller does before topk_unit.
template <int CMAX> struct TopkKeys {
    uint32_t key[CMAX];
    float raw[CMAX];
};

template <int NT, int CMAX>
__device__ __forceinline__ void topk_load(const float *__restrict__ s, int NB, TopkKeys<CMAX> &k) {
    const int C = (NB + NT - 1) / NT;
    const int begin = threadIdx.x * C;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        const int id = begin + i;
        k.raw[i] = (i < C && id < NB) ? s[id] : 0.f;
    }
}

template <int NT, int CMAX>
__device__ void topk_unit(TopkKeys<CMAX> &kk, int NB, int K, int32_t *__restrict__ out,
                          int32_t *__restrict__ out2, int32_t *out_lds,
                          uint32_t *__restrict__ err) {
    constexpr int NW = NT / 64;
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t red_mx[NW], red_mn[NW];
    __shared__ int pick[2][3];  // digit, keys above the digit's bin, keys in the bin
    __shared__ int wave_cnt[NW];
    __shared__ int scan_a[NW];
    __shared__ __attribute__((aligned(16))) uint32_t ckey[kTopkMaxK];
    __shared__ __attribute__((aligned(16))) int32_t cid[kTopkMaxK];
    __shared__ int rank_sh[kTopkMaxK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Kp = K < NB ? K : NB;
    if (Kp <= 0) {
        for (int i = tid; i < K; i += NT) {
            out[i] = -1;
            if (out2) out2[i] = -1;
            if (out_lds) out_lds[i] = -1;
        }
        return;
    }

    const int C = (NB + NT - 1) / NT;
    const int begin = tid * C;
    uint32_t *key = kk.key;
    bool bad = false;
    uint32_t lmx = 0u, lmn = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        const int id = begin + i;
        const bool valid = i < C && id < NB;
        key[i] = valid ? order_key(kk.raw[i], bad) : 0u;
        if (valid) {
            lmx = key[i] > lmx ? key[i] : lmx;
            lmn = key[i] < lmn ? key[i] : lmn;
        }
    }
    if (bad) atomicOr(err, kErrNonFinite);
    lmx = wave_max_u32(lmx);
    lmn = wave_min_u32(lmn);
    if (lane == 0) {
        red_mx[wave] = lmx;
        red_mn[wave] = lmn;
    }
    for (int i = tid; i < Kp; i += NT) rank_sh[i] = 0;
    for (int i = tid; i < 256; i += NT) hist[0][i] = 0u;
    __syncthreads();
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kmax = red_mx[w] > kmax ? red_mx[w] : kmax;
        kmin = red_mn[w] < kmin ? red_mn[w] : kmin;
    }

    // bits at and above `hi` are fixed to those of `prefix`; `need` keys are
    // still to be taken among the keys that match them
    const uint32_t diff = kmax ^ kmin;
    int hi = diff ? 32 - __builtin_clz(diff) : 0;
    uint32_t prefix = hi >= 32 ? 0u : (kmax & ~((1u << hi) - 1u));
    int need = Kp;
    bool exact = false;
    int cur = 0;
    while (hi > 0 && !exact) {
        const int width = hi < 8 ? hi : 8;
        const int sh = hi - width;
        const uint32_t fixed = hi >= 32 ? 0u : ~((1u << hi) - 1u);
        // hist[cur] was cleared before the previous barrier; the other
        // buffer, read by the previous pass's scan, is cleared for the next
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            if (i < C && id < NB && (key[i] & fixed) == prefix)
                atomicAdd(&hist[cur][(key[i] >> sh) & ((1u << width) - 1u)], 1u);
        }
        for (int i = tid; i < 256; i += NT) hist[cur ^ 1][i] = 0u;
        __syncthreads();
        if (wave == 0) {
            // suffix sums over the 256 bins, four per lane, highest digit first
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = hist[cur][4 * lane + j];
            const uint32_t mine = h[0] + h[1] + h[2] + h[3];
            const uint32_t suf = wave_suffix_sum_u32(mine);  // lanes >= this one
            uint32_t above = suf - mine;
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                if (above < (uint32_t)need && above + h[j] >= (uint32_t)need) {
                    pick[cur][0] = 4 * lane + j;
                    pick[cur][1] = (int)above;
                    pick[cur][2] = (int)h[j];
                }
                above += h[j];
            }
        }
        __syncthreads();
        const int digit = pick[cur][0];
        need -= pick[cur][1];
        prefix |= (uint32_t)digit << sh;
        hi = sh;
        exact = pick[cur][2] == need;
        cur ^= 1;
    }
    // selection: keys >= prefix when exact; otherwise keys > tau = prefix and
    // the `need` lowest-id keys equal to tau
    const uint32_t tau = prefix;
    int eq_before = 0;
    if (!exact) {
        int eq = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            eq += (i < C && id < NB && key[i] == tau) ? 1 : 0;
        }
        eq_before = block_excl_scan<NT>(eq, scan_a);
    }
    bool take[CMAX];
    int my_takes = 0;
    {
        int eq_seen = 0;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            bool t = false;
            if (i < C && id < NB) {
                if (exact) {
                    t = key[i] >= tau;
                } else {
                    t = key[i] > tau;
                    if (key[i] == tau) {
                        t = eq_before + eq_seen < need;
                        ++eq_seen;
                    }
                }
            }
            take[i] = t;
            my_takes += t ? 1 : 0;
        }
    }
    // compaction: wave bases through LDS, lane positions through ballots
    const uint32_t wt = wave_add_u32((uint32_t)my_takes);
    if (lane == 0) wave_cnt[wave] = (int)wt;
    __syncthreads();
    int pos = 0;
    for (int w = 0; w < wave; ++w) pos += wave_cnt[w];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        const unsigned long long b = __ballot(take[i]);
        if (take[i]) {
            const int p = pos + lanes_below(b);
            if (p < kTopkMaxK) {
                ckey[p] = key[i];
                cid[p] = begin + i;
            }
        }
        pos += __popcll(b);
    }
    __syncthreads();

    if (Kp <= 128) {
        // one wave sorts the winners: 64-bit composites (key, ~id) in
        // descending order are (score desc, id asc); two per lane, element
        // e * 64 + lane, bitonic network, cross-lane pairs through DPP and
        // shuffles
        if (wave == 0) {
            unsigned long long v[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = e * 64 + lane;
                v[e] = i < Kp ? ((unsigned long long)ckey[i] << 32) | (uint32_t)~(uint32_t)cid[i]
                              : 0ull;  // sorts last: no finite score has key 0
            }
            // k = 2^kk is the size of the sorted runs being merged, j = 2^jj the
            // compare distance; distances below 16 exchange through DPP
            static_for<1, 8>([&](auto kkI) {
                constexpr int kk = decltype(kkI)::value, k = 1 << kk;
                static_for<0, kk>([&](auto tI) {
                    constexpr int j = 1 << (kk - 1 - decltype(tI)::value);
                    if constexpr (j == 64) {  // partner is the lane's other element
                        // element 0 has bit 64 clear: it keeps the larger
                        // value when the block (bit k = 128) sorts descending
                        const unsigned long long a = v[0], b = v[1];
                        v[0] = a > b ? a : b;
                        v[1] = a > b ? b : a;
                    } else {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int i = e * 64 + lane;
                            const unsigned long long o = lane_xor_u64<j>(v[e]);
                            // descending overall: the pair's lower index keeps the
                            // larger value in blocks with (i & k) == 0
                            const bool lower = (i & j) == 0;
                            const bool desc = (i & k) == 0;
                            const bool keep_max = lower == desc;
                            v[e] = keep_max ? (v[e] > o ? v[e] : o) : (v[e] < o ? v[e] : o);
                        }
                    }
                });
            });
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = e * 64 + lane;
                if (r < Kp) {
                    const int32_t id = (int32_t)~(uint32_t)v[e];
                    out[r] = id;
                    if (out2) out2[r] = id;
                    if (out_lds) out_lds[r] = id;
                }
            }
        }
        for (int i = Kp + tid; i < K; i += NT) {
            out[i] = -1;
            if (out2) out2[i] = -1;
            if (out_lds) out_lds[i] = -1;
        }
        return;
    }

    // place each winner by counting the winners that order before it; two
    // threads share a winner when there are enough threads
    const int parts = (NT >= 2 * Kp) ? 2 : 1;
    const int span = (Kp + parts - 1) / parts;
    for (int idx = tid; idx < Kp * parts; idx += NT) {
        const int i = idx % Kp, part = idx / Kp;
        const uint32_t ki = ckey[i];
        const int32_t ii = cid[i];
        auto before = [&](uint32_t kj, int32_t ij) { return (kj > ki || (kj == ki && ij < ii)) ? 1 : 0; };
        int j = part * span;
        const int j1 = (j + span) < Kp ? (j + span) : Kp;
        int rank = 0;
        for (; j < j1 && (j & 3); ++j) rank += before(ckey[j], cid[j]);
#pragma unroll 4
        for (; j + 8 <= j1; j += 8) {
            const uint4 ka = *reinterpret_cast<const uint4 *>(ckey + j);
            const uint4 kb = *reinterpret_cast<const uint4 *>(ckey + j + 4);
            const int4 ia = *reinterpret_cast<const int4 *>(cid + j);
            const int4 ib = *reinterpret_cast<const int4 *>(cid + j + 4);
            rank += before(ka.x, ia.x) + before(ka.y, ia.y) + before(ka.z, ia.z) +
                    before(ka.w, ia.w) + before(kb.x, ib.x) + before(kb.y, ib.y) +
                    before(kb.z, ib.z) + before(kb.w, ib.w);
        }
        for (; j < j1; ++j) rank += before(ckey[j], cid[j]);
        if (parts == 1) rank_sh[i] = rank;
        else atomicAdd(&rank_sh[i], rank);
    }
    __syncthreads();
    for (int i = tid; i < Kp; i += NT) {
        const int32_t id = cid[i];
        const int r = rank_sh[i];
        out[r] = id;
        if (out2) out2[r] = id;
        if (out_lds) out_lds[r] = id;
    }
    for (int i = Kp + tid; i < K; i += NT) {
        out[i] = -1;
        if (out2) out2[i] = -1;
        if (out_lds) out_lds[i] = -1;
    }
}

template <int NT, int CMAX>
__global__ __launch_bounds__(NT) void topk_kernel(const float *__restrict__ scores, int64_t NBmax,
                                                  int NB, int K, int32_t *__restrict__ ids,
                                                  int32_t *__restrict__ ids_copy,
                                                  uint32_t *__restrict__ err) {
    const int64_t u = blockIdx.x;
    TopkKeys<CMAX> kk;
    topk_load<NT, CMAX>(scores + u * NBmax, NB, kk);
    topk_unit<NT, CMAX>(kk, NB, K, ids + u * K, ids_copy ? ids_copy + u * K : nullptr, nullptr,
                        err);
}

// Hash of a block id for the LDS residency table.
__device__ __forceinline__ uint32_t block_hash(int32_t blk) {
    return ((uint32_t)blk * 2654435761u) >> 8;
}

// Slots of the LDS residency hash: a power of two of at least twice S, so a
// probe sequence always meets an empty slot.
__host__ __device__ constexpr int hash_size(int S) {
    int h = 64;
    while (h < 2 * S) h *= 2;
    return h;
}

// Resident-block lookup in LDS: up to this many blocks a direct table
// slot_of[block] (int16, S <= 2048), one read per lookup; past it a hash of
// the resident blocks with linear probing.
constexpr int64_t kDirectMax = 16384;

// 32-bit words of LDS the lookup table takes (16-byte multiple).
__host__ __device__ constexpr int table_ints(int S, int64_t NB) {
    return NB <= kDirectMax ? (int)(((NB + 7) / 8) * 4) : 2 * hash_size(S);
}

// Bytes of LDS scratch select_unit needs.
__host__ __device__ constexpr size_t select_lds_bytes(int K, int S) {
    return sizeof(int32_t) * (3 * (size_t)K + 2 * (size_t)S + 2) +
           sizeof(unsigned long long) * ((size_t)S + 1);
}

// Diff / cap / LRU of unit u, run by the 64 lanes of one wave.  sel: the K
// selected ids (global or LDS); sb_in / lu_in: the slot tables to read (the
// global tables, or LDS copies of them); the global tables slot_block /
// last_used / block_slot (rows of unit u) are written.  sh: LDS scratch of
// select_lds_bytes(K, S).
__device__ void select_unit(int64_t u, const int32_t *sel, const int32_t *sb_in,
                            const int32_t *lu_in, int32_t *__restrict__ slot_block,
                            int32_t *__restrict__ last_used, int32_t *__restrict__ block_slot,
                            int K, int S, int64_t NBmax, int cap, int32_t t,
                            int32_t *__restrict__ fetch_block, int32_t *__restrict__ fetch_slot,
                            int32_t *__restrict__ att_block, int32_t *__restrict__ att_slot,
                            int32_t *__restrict__ counts, DevStats *stats, uint32_t *err,
                            int32_t *sh, const int16_t *slot_of, const int32_t *hkey,
                            const int32_t *hval, uint32_t hmask, int attend_all) {
    int32_t *hit_blk = sh;             // [K]
    int32_t *hit_slot = hit_blk + K;   // [K]
    int32_t *miss_blk = hit_slot + K;  // [K]
    int32_t *cand = miss_blk + K;      // [S] slots to fill, in order
    int32_t *selected = cand + S;      // [S] slot holds a selected block
    unsigned long long *vkey = reinterpret_cast<unsigned long long *>(selected + S + (K & 1));  // 8-byte aligned

    const int lane = threadIdx.x & 63;
    int32_t *sb = slot_block + u * S;
    int32_t *lu = last_used + u * S;
    int32_t *bs = block_slot + u * NBmax;

    for (int s = lane; s < S; s += 64) selected[s] = 0;
    wave_sync();

    // hits and misses, in top-K order
    int nh = 0, nm = 0;
    for (int base = 0; base < K; base += 64) {
        const int i = base + lane;
        const int32_t id = i < K ? sel[i] : -1;
        int32_t s = -1;
        if (id >= 0) {
            if (slot_of) {  // LDS table of the resident blocks
                s = slot_of[id];
            } else if (hkey) {  // LDS hash of the resident blocks: linear probing
                uint32_t hh = block_hash(id) & hmask;
                while (true) {
                    const int32_t k = hkey[hh];
                    if (k == id) {
                        s = hval[hh];
                        break;
                    }
                    if (k < 0) break;
                    hh = (hh + 1) & hmask;
                }
            } else {
                s = bs[id];
            }
        }
        const bool hit = id >= 0 && s >= 0;
        const bool miss = id >= 0 && s < 0;
        const unsigned long long hb = __ballot(hit), mb = __ballot(miss);
        if (hit) {
            const int p = nh + lanes_below(hb);
            hit_blk[p] = id;
            hit_slot[p] = s;
            selected[s] = 1;
        }
        if (miss) miss_blk[nm + lanes_below(mb)] = id;
        nh += __popcll(hb);
        nm += __popcll(mb);
    }
    wave_sync();
    const int n = nm < cap ? nm : cap;

    // empty slots first, ascending; then LRU victims among held, non-selected
    int nfree = 0;
    for (int base = 0; base < S; base += 64) {
        const int s = base + lane;
        const bool fr = s < S && sb_in[s] < 0;
        const unsigned long long fb = __ballot(fr);
        if (fr) cand[nfree + lanes_below(fb)] = s;
        nfree += __popcll(fb);
    }
    for (int s = lane; s < S; s += 64) {
        const int32_t blk = sb_in[s];
        vkey[s] = (blk >= 0 && !selected[s])
                      ? ((unsigned long long)((uint32_t)lu_in[s] ^ 0x80000000u) << 32) |
                            (uint32_t)blk
                      : ~0ull;
    }
    wave_sync();
    const int need = n - nfree;
    if (need > 0 && need <= 16 && S <= 256) {
        // pick the `need` least-recent victims by repeated wave minimum over
        // (last_used, block) keys held in registers (at most 4 per lane)
        unsigned long long mine[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) mine[k] = (lane + 64 * k < S) ? vkey[lane + 64 * k] : ~0ull;
        for (int r = 0; r < need; ++r) {
            unsigned long long lo = mine[0];
#pragma unroll
            for (int k = 1; k < 4; ++k) lo = mine[k] < lo ? mine[k] : lo;
            const uint32_t hi_min = wave_min_u32((uint32_t)(lo >> 32));
            const uint32_t lo_min = wave_min_u32((uint32_t)(lo >> 32) == hi_min ? (uint32_t)lo
                                                                                : 0xFFFFFFFFu);
            const unsigned long long best = ((unsigned long long)hi_min << 32) | lo_min;
            if (best == ~0ull) break;  // fewer victims than needed: reported below
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (mine[k] == best) {
                    cand[nfree + r] = lane + 64 * k;
                    mine[k] = ~0ull;
                }
        }
    } else if (need > 0) {
        for (int s = lane; s < S; s += 64) {
            const unsigned long long k = vkey[s];
            if (k == ~0ull) continue;
            int rank = 0;
            for (int r = 0; r < S; ++r) rank += vkey[r] < k ? 1 : 0;
            if (rank < need) cand[nfree + rank] = s;
        }
    }
    wave_sync();
    int nvict = 0;
    for (int s = lane; s < S; s += 64) nvict += vkey[s] != ~0ull ? 1 : 0;
    nvict = wave_sum_i(nvict);
    if (nfree + nvict < n) {  // cannot happen with S >= K
        // tables untouched; the lists of this step are empty, so the next
        // attention attends nothing instead of the previous step's list
        if (lane == 0) {
            atomicOr(err, kErrSlots);
            counts[u * 4 + 0] = 0;
            counts[u * 4 + 1] = 0;
            counts[u * 4 + 2] = 0;
            counts[u * 4 + 3] = nm;
        }
        return;
    }

    // apply: evict, fill, refresh recency, emit lists
    int32_t *fb = fetch_block + u * K, *fs = fetch_slot + u * K;
    int32_t *ab = att_block + u * K, *as = att_slot + u * K;
    for (int i = lane; i < n; i += 64) {
        const int s = cand[i];
        const int32_t old = sb_in[s];
        if (old >= 0) bs[old] = -1;
    }
    // attend-all reading: the held blocks that stay and were not selected
    int nr = 0;
    if (attend_all) {
        for (int i = lane; i < n; i += 64) selected[cand[i]] = 2;  // refilled
        wave_sync();
        for (int base = 0; base < S; base += 64) {
            const int s = base + lane;
            const bool keep = s < S && sb_in[s] >= 0 && selected[s] == 0;
            const unsigned long long kb = __ballot(keep);
            if (keep) {
                const int p = nh + nr + lanes_below(kb);
                ab[p] = sb_in[s];
                as[p] = s;
            }
            nr += __popcll(kb);
        }
    }
    wave_sync();
    for (int i = lane; i < n; i += 64) {
        const int s = cand[i];
        const int32_t blk = miss_blk[i];
        sb[s] = blk;
        bs[blk] = s;
        lu[s] = t;
        fb[i] = blk;
        fs[i] = s;
        ab[nh + nr + i] = blk;
        as[nh + nr + i] = s;
    }
    for (int i = lane; i < nh; i += 64) {
        lu[hit_slot[i]] = t;
        ab[i] = hit_blk[i];
        as[i] = hit_slot[i];
    }
    if (lane == 0) {
        counts[u * 4 + 0] = nh + nr + n;
        counts[u * 4 + 1] = nh;
        counts[u * 4 + 2] = n;
        counts[u * 4 + 3] = nm;
        // the unit's own counters: one workgroup per unit and the handle's
        // selects run in order, so no atomics (1,024 same-address atomics per
        // launch at 256 units held the kernel's end for microseconds)
        DevStats &su = stats[u];
        su.hits += (unsigned long long)nh;
        su.misses += (unsigned long long)nm;
        su.fetched += (unsigned long long)n;
        su.attended += (unsigned long long)(nh + nr + n);
    }
}

__global__ __launch_bounds__(64) void select_kernel(
    const int32_t *__restrict__ ids, int32_t *__restrict__ slot_block,
    int32_t *__restrict__ last_used, int32_t *__restrict__ block_slot, int K, int S,
    int64_t NBmax, int cap, int32_t t, int32_t *__restrict__ fetch_block,
    int32_t *__restrict__ fetch_slot, int32_t *__restrict__ att_block,
    int32_t *__restrict__ att_slot, int32_t *__restrict__ counts, DevStats *stats,
    uint32_t *err, int attend_all) {
    extern __shared__ __attribute__((aligned(16))) int32_t sh[];
    const int64_t u = blockIdx.x;
    select_unit(u, ids + u * K, slot_block + u * S, last_used + u * S, slot_block, last_used,
                block_slot, K, S, NBmax, cap, t, fetch_block, fetch_slot, att_block, att_slot,
                counts, stats, err, sh, nullptr, nullptr, nullptr, 0u, attend_all);
}

// Top-K and select of one unit in one workgroup.
template <int NT, int CMAX>
__global__ __launch_bounds__(NT) void topk_select_kernel(
    const float *__restrict__ scores, int NB, int32_t *__restrict__ ids,
    int32_t *__restrict__ slot_block, int32_t *__restrict__ last_used,
    int32_t *__restrict__ block_slot, int K, int S, int64_t NBmax, int cap, int32_t t,
    int32_t *__restrict__ fetch_block, int32_t *__restrict__ fetch_slot,
    int32_t *__restrict__ att_block, int32_t *__restrict__ att_slot,
    int32_t *__restrict__ counts, DevStats *stats, uint32_t *err, int attend_all) {
    extern __shared__ __attribute__((aligned(16))) int32_t sh[];
    const int64_t u = blockIdx.x;
    const int K4 = (K + 3) & ~3, S4 = (S + 3) & ~3;
    const int HS = hash_size(S);
    int32_t *sel_lds = sh;                 // [K]
    int32_t *sb_lds = sel_lds + K4;        // [S]
    int32_t *lu_lds = sb_lds + S4;         // [S]
    // resident block -> slot: a direct table, or a hash past kDirectMax blocks
    const bool direct = NB <= kDirectMax;
    int32_t *tab = lu_lds + S4;
    int16_t *slot_of = direct ? reinterpret_cast<int16_t *>(tab) : nullptr;
    int32_t *hkey = direct ? nullptr : tab;    // [HS]
    int32_t *hval = direct ? nullptr : tab + HS;
    int32_t *scratch = tab + table_ints(S, NB);  // 16-byte aligned
    // the scores are read while the tables below are read and indexed
    TopkKeys<CMAX> kk;
    topk_load<NT, CMAX>(scores + u * NBmax, NB, kk);
    if (direct) {
        for (int i = threadIdx.x; i < NB; i += NT) slot_of[i] = -1;
    } else {
        for (int i = threadIdx.x; i < HS; i += NT) hkey[i] = -1;
    }
    __syncthreads();
    // tables into LDS and the resident blocks into the lookup table, while the top-K
    // below still waits for its scores
    for (int s = threadIdx.x; s < S; s += NT) {
        const int32_t blk = slot_block[u * S + s];
        sb_lds[s] = blk;
        lu_lds[s] = last_used[u * S + s];
        if (blk >= 0 && blk < NB) {  // blocks past NB are never selected
            if (direct) {
                slot_of[blk] = (int16_t)s;
            } else {
                uint32_t hh = block_hash(blk) & (uint32_t)(HS - 1);
                while (atomicCAS(&hkey[hh], -1, blk) != -1) hh = (hh + 1) & (uint32_t)(HS - 1);
                hval[hh] = s;
            }
        }
    }
    topk_unit<NT, CMAX>(kk, NB, K, ids + u * K, nullptr, sel_lds, err);
    __syncthreads();
    if (threadIdx.x < 64)
        select_unit(u, sel_lds, sb_lds, lu_lds, slot_block, last_used, block_slot, K, S, NBmax,
                    cap, t, fetch_block, fetch_slot, att_block, att_slot, counts, stats, err,
                    scratch, slot_of, hkey, hval, (uint32_t)(HS - 1), attend_all);
}

// Score, top-K and select of one unit in one workgroup (NT / 64 waves): the
// unit's tiles are scored into LDS by the first nws waves (the slot tables are
// indexed meanwhile), copied out for inspection, and the top-K and select run
// on the LDS copy: no score round trip through HBM and one launch instead of
// two.  The summary read is the same as the score kernel's.
template <int D, int QT, int CMAX, int NT, bool XT>
__global__ __launch_bounds__(NT) void score_topk_select_kernel(
    const uint16_t *__restrict__ summ, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ drafts, int n_drafts, int qskip, float *__restrict__ scores,
    int B, int Hq, int Hkv, int G, int64_t unit_elems, int NB, int32_t *__restrict__ ids,
    int32_t *__restrict__ slot_block, int32_t *__restrict__ last_used,
    int32_t *__restrict__ block_slot, int K, int S, int64_t NBmax, int cap, int32_t t,
    int32_t *__restrict__ fetch_block, int32_t *__restrict__ fetch_slot,
    int32_t *__restrict__ att_block, int32_t *__restrict__ att_slot,
    int32_t *__restrict__ counts, DevStats *stats, uint32_t *err, int attend_all, int nws) {
    constexpr int NW = NT / 64;
    extern __shared__ __attribute__((aligned(16))) int32_t sh[];
    const int64_t u = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K4 = (K + 3) & ~3, S4 = (S + 3) & ~3;
    const int HS = hash_size(S);
    int32_t *sel_lds = sh;                 // [K]
    int32_t *sb_lds = sel_lds + K4;        // [S]
    int32_t *lu_lds = sb_lds + S4;         // [S]
    // resident block -> slot: a direct table, or a hash past kDirectMax blocks
    const bool direct = NB <= kDirectMax;
    int32_t *tab = lu_lds + S4;
    int16_t *slot_of = direct ? reinterpret_cast<int16_t *>(tab) : nullptr;
    int32_t *hkey = direct ? nullptr : tab;    // [HS]
    int32_t *hval = direct ? nullptr : tab + HS;
    int32_t *scratch = tab + table_ints(S, NB);  // 16-byte aligned
    float *sc = reinterpret_cast<float *>(scratch + ((select_lds_bytes(K, S) + 15) / 16) * 4);
    const int h = (int)(u % Hkv), b = (int)(u / Hkv);
    const int ntiles = (NB + 31) / 32;

    const int NWS = nws < NW ? nws : NW;
    ScoreTiles<D, QT> st;
    st.setup(summ, u, unit_elems);
    int tile = wave < NWS ? wave : ntiles;
    // XT, as in the score kernel: a wave owning one tile more than the fewest
    // loads that last tile now into a second buffer (with one workgroup per
    // CU only: the buffer's registers would keep other kernels' waves off)
    const int mine = tile < ntiles ? (ntiles - tile + NWS - 1) / NWS : 0;
    const bool extra = XT && mine >= 2 && mine > ntiles / NWS;
    const int t_stop = extra ? tile + NWS * (mine - 1) : ntiles;
    bf16x8 bx[XT ? ScoreTiles<D, QT>::NI : 1];
    if (tile < ntiles) st.load(tile);  // in flight while the tables are indexed
    if constexpr (XT) {
        if (extra) st.load_to(bx, t_stop);
    }
    if (direct) {
        for (int i = threadIdx.x; i < NB; i += NT) slot_of[i] = -1;
    } else {
        for (int i = threadIdx.x; i < HS; i += NT) hkey[i] = -1;
    }
    __syncthreads();
    for (int s = threadIdx.x; s < S; s += NT) {
        const int32_t blk = slot_block[u * S + s];
        sb_lds[s] = blk;
        lu_lds[s] = last_used[u * S + s];
        if (blk >= 0 && blk < NB) {  // blocks past NB are never selected
            if (direct) {
                slot_of[blk] = (int16_t)s;
            } else {
                uint32_t hh = block_hash(blk) & (uint32_t)(HS - 1);
                while (atomicCAS(&hkey[hh], -1, blk) != -1) hh = (hh + 1) & (uint32_t)(HS - 1);
                hval[hh] = s;
            }
        }
    }
    if (wave < NWS) {
        st.rows(q, drafts, n_drafts, qskip, B, Hq, G, b, h);
        for (; tile < t_stop; tile += NWS) {
            const float best = st.best();
            if (st.half == 0) sc[tile * 32 + st.m] = best;
            if (tile + NWS < t_stop) st.load(tile + NWS);
        }
        if constexpr (XT) {
            if (extra) {
                const float best = st.best_of(bx);
                if (st.half == 0) sc[t_stop * 32 + st.m] = best;
            }
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < NB; j += NT) scores[u * NBmax + j] = sc[j];
    TopkKeys<CMAX> kk;
    {
        const int C = (NB + NT - 1) / NT;
        const int begin = threadIdx.x * C;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int id = begin + i;
            kk.raw[i] = (i < C && id < NB) ? sc[id] : 0.f;
        }
    }
    topk_unit<NT, CMAX>(kk, NB, K, ids + u * K, nullptr, sel_lds, err);
    __syncthreads();
    if (threadIdx.x < 64)
        select_unit(u, sel_lds, sb_lds, lu_lds, slot_block, last_used, block_slot, K, S, NBmax,
                    cap, t, fetch_block, fetch_slot, att_block, att_slot, counts, stats, err,
                    scratch, slot_of, hkey, hval, (uint32_t)(HS - 1), attend_all);
}

__global__ __launch_bounds__(64) void evict_kernel(const int32_t *__restrict__ blocks,
                                                   const int32_t *__restrict__ counts,
                                                   int max_per_unit, int32_t *slot_block,
                                                   int32_t *block_slot, int S, int64_t NBmax) {
    const int64_t u = blockIdx.x;
    const int n = counts[u];
    for (int i = threadIdx.x; i < n && i < max_per_unit; i += 64) {
        const int32_t blk = blocks[u * max_per_unit + i];
        if (blk < 0 || blk >= NBmax) continue;
        const int32_t s = block_slot[u * NBmax + blk];
        if (s < 0) continue;
        slot_block[u * S + s] = -1;
        block_slot[u * NBmax + blk] = -1;
    }
}

// Forced non-residency from seeded draws: unit u empties the slots of
// floor(fraction * n_att) entries of its last attended list, the entries whose
// draws[u][i] are smallest (ties to the lower list position); recency is left
// as it is.  The count uses a separately rounded product and sum (no fused
// multiply-add), as the draws' consumer on the host computes it.
__global__ __launch_bounds__(256) void evict_attended_kernel(
    const double *__restrict__ draws, double fraction, const int32_t *__restrict__ att_block,
    const int32_t *__restrict__ counts, int32_t *__restrict__ slot_block,
    int32_t *__restrict__ block_slot, int K, int S, int64_t NBmax) {
    __shared__ double dr[1024];
    const int64_t u = blockIdx.x;
    const int na = __builtin_amdgcn_readfirstlane(counts[u * 4]);
    const int n = (int)floor(__dadd_rn(__dmul_rn(fraction, (double)na), 1e-9));
    if (n <= 0) return;
    for (int i = threadIdx.x; i < na; i += 256) dr[i] = draws[u * K + i];
    __syncthreads();
    for (int i = threadIdx.x; i < na; i += 256) {
        const double di = dr[i];
        int rank = 0;
        for (int j = 0; j < na; ++j) {
            const double dj = dr[j];
            rank += (dj < di || (dj == di && j < i)) ? 1 : 0;
        }
        if (rank >= n) continue;
        const int32_t blk = att_block[u * K + i];
        if (blk < 0 || blk >= NBmax) continue;
        const int32_t s = block_slot[u * NBmax + blk];
        if (s < 0) continue;
        slot_block[u * S + s] = -1;
        block_slot[u * NBmax + blk] = -1;
    }
}

__global__ __launch_bounds__(256) void rebuild_block_slot_kernel(
    const int32_t *__restrict__ slot_block, int32_t *__restrict__ block_slot, int S,
    int64_t NBmax) {
    const int64_t u = blockIdx.y;
    for (int64_t j = blockIdx.x * 256LL + threadIdx.x; j < NBmax; j += gridDim.x * 256LL)
        block_slot[u * NBmax + j] = -1;
    __syncthreads();
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s < S; s += 256) {
            const int32_t blk = slot_block[u * S + s];
            if (blk >= 0) block_slot[u * NBmax + blk] = s;
        }
}

// Workgroup size and per-thread key capacity of the top-K for NB blocks.
// Each thread holds C = ceil(NB / NT) keys in registers; the loops run over
// the compiled capacity CMAX, and their cost follows CMAX rather than C
// (measured: 2,049 blocks take 7.0 us with 256 threads x 16 keys, 6.0 us with
// 1,024 x 4; 8,193 blocks 19 us with 256 x 64, 10.6 us with 1,024 x 16).  So
// the thread count grows first and C fits a power of two.  NB <= 65,536.
static int topk_threads(int64_t NB) { return NB <= 1024 ? 256 : NB <= 2048 ? 512 : 1024; }

#define OASIS_TOPK_DISPATCH(NB, LAUNCH)                        \
    do {                                                       \
        const int nt_ = topk_threads(NB);                      \
        const int64_t c_ = ((NB) + nt_ - 1) / nt_;             \
        if (nt_ == 256) LAUNCH(256, 4);                        \
        else if (nt_ == 512) LAUNCH(512, 4);                   \
        else if (c_ <= 4) LAUNCH(1024, 4);                     \
        else if (c_ <= 8) LAUNCH(1024, 8);                     \
        else if (c_ <= 16) LAUNCH(1024, 16);                   \
        else if (c_ <= 32) LAUNCH(1024, 32);                   \
        else LAUNCH(1024, 64);                                 \
    } while (0)

hipError_t launch_topk(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                       int32_t *ids_copy, uint32_t *err, hipStream_t st) {
    dim3 grid((unsigned)D.units());
#define OASIS_TOPK(NT_, CM_)                                                                    \
    OASIS_LAUNCH((topk_kernel<NT_, CM_>), grid, dim3(NT_), 0, st, scores, D.NBmax,      \
                       (int)NB, D.K, ids, ids_copy, err)
    OASIS_TOPK_DISPATCH(NB, OASIS_TOPK);
#undef OASIS_TOPK
    return hipGetLastError();
}

hipError_t launch_select(const Dims &D, const int32_t *ids, int32_t *slot_block,
                         int32_t *last_used, int32_t *block_slot, int cap, int32_t t,
                         int32_t *fetch_block, int32_t *fetch_slot, int32_t *att_block,
                         int32_t *att_slot, int32_t *counts, DevStats *stats, uint32_t *err,
                         hipStream_t st) {
    OASIS_LAUNCH(select_kernel, dim3((unsigned)D.units()), dim3(64),
                       select_lds_bytes(D.K, D.S), st, ids, slot_block, last_used, block_slot,
                       D.K, D.S, D.NBmax, cap, t, fetch_block, fetch_slot, att_block, att_slot,
                       counts, stats, err, D.attend_all ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_topk_select(const Dims &D, const float *scores, int64_t NB, int32_t *ids,
                              int32_t *slot_block, int32_t *last_used, int32_t *block_slot,
                              int cap, int32_t t, int32_t *fetch_block, int32_t *fetch_slot,
                              int32_t *att_block, int32_t *att_slot, int32_t *counts,
                              DevStats *stats, uint32_t *err, hipStream_t st) {
    dim3 grid((unsigned)D.units());
    const size_t lds = sizeof(int32_t) * ((size_t)((D.K + 3) & ~3) + 2 * (size_t)((D.S + 3) & ~3) +
                                          (size_t)table_ints(D.S, NB)) +
                       select_lds_bytes(D.K, D.S);
    if (lds > 64 * 1024) {  // large pools: the two kernels one after the other
        hipError_t e = launch_topk(D, scores, NB, ids, nullptr, err, st);
        if (e != hipSuccess) return e;
        return launch_select(D, ids, slot_block, last_used, block_slot, cap, t, fetch_block,
                             fetch_slot, att_block, att_slot, counts, stats, err, st);
    }
#define OASIS_TS(NT_, CM_)                                                                      \
    OASIS_LAUNCH((topk_select_kernel<NT_, CM_>), grid, dim3(NT_), lds, st, scores,      \
                       (int)NB, ids, slot_block, last_used, block_slot, D.K, D.S, D.NBmax, cap, \
                       t, fetch_block, fetch_slot, att_block, att_slot, counts, stats, err,      \
                       D.attend_all ? 1 : 0)
    OASIS_TOPK_DISPATCH(NB, OASIS_TS);
#undef OASIS_TS
    return hipGetLastError();
}

static size_t fused_lds_bytes(const Dims &D, int64_t NB) {
    const size_t ints = (size_t)((D.K + 3) & ~3) + 2 * (size_t)((D.S + 3) & ~3) +
                        (size_t)table_ints(D.S, NB);
    return sizeof(int32_t) * ints + ((select_lds_bytes(D.K, D.S) + 15) / 16) * 16 +
           sizeof(float) * 32 * (size_t)((NB + 31) / 32);
}

bool score_topk_fusable(const Dims &D, int64_t NB, int n_rows) {
    // one workgroup per unit must still fill the GPU, and the unit's scores
    // must fit in LDS next to the select's tables
    return D.tiled && D.d == 128 && n_rows <= 128 && D.units() >= compute_units(D) && NB >= 1 &&
           NB <= 8192 && fused_lds_bytes(D, NB) <= 64 * 1024;
}

hipError_t launch_score_topk_select(const Dims &D, const void *summ, const void *q,
                                    const void *drafts, int n_drafts, int64_t NB, float *scores,
                                    int32_t *ids, int32_t *slot_block, int32_t *last_used,
                                    int32_t *block_slot, int cap, int32_t t,
                                    int32_t *fetch_block, int32_t *fetch_slot,
                                    int32_t *att_block, int32_t *att_slot, int32_t *counts,
                                    DevStats *stats, uint32_t *err, hipStream_t st) {
    const int qskip = q ? 0 : 1;
    const int Q = D.G * (1 - qskip + n_drafts);
    if (!score_topk_fusable(D, NB, Q)) return hipErrorInvalidValue;
    const int QT = (Q + 31) / 32;
    const size_t lds = fused_lds_bytes(D, NB);
    const dim3 grid((unsigned)D.units());
    // 8 waves once the keys outgrow 8 per thread, where the query rows leave
    // the registers for it (at most two 32-row MFMA tiles)
    const int nt = (QT <= 2 && NB > 2048) ? 512 : 256;
    // Scoring waves: with one workgroup per CU, four (one 16 KB tile stream
    // per SIMD, as in the score kernel) read the summaries faster than eight
    // (51.6 against 53.6 us on the Qwen3-8B layer); with two or more per CU
    // every wave scores (10.30 against 10.83 ms per 36-layer step, where the
    // kernel shares the GPU with other layers' attention).
    const int nws = D.units() <= compute_units(D) ? 4 : nt / 64;
    const int C = (int)((NB + nt - 1) / nt);
    const bool xt = nws == 4 && QT == 1;  // one workgroup per CU
#define OASIS_STS_X(QT_, CM_, NT_, XT_)                                                          \
    OASIS_LAUNCH((score_topk_select_kernel<128, QT_, CM_, NT_, XT_>), grid, dim3(NT_), lds, st,  \
                 (const uint16_t *)summ, (const uint16_t *)q, (const uint16_t *)drafts, n_drafts, \
                 qskip, scores, D.B, D.Hq, D.Hkv, D.G, D.summ_unit_elems(), (int)NB, ids,         \
                 slot_block, last_used, block_slot, D.K, D.S, D.NBmax, cap, t, fetch_block,       \
                 fetch_slot, att_block, att_slot, counts, stats, err, D.attend_all ? 1 : 0, nws)
#define OASIS_STS(QT_, CM_, NT_)                                                                 \
    do {                                                                                         \
        if (QT_ == 1 && xt) OASIS_STS_X(QT_, CM_, NT_, true);                                    \
        else OASIS_STS_X(QT_, CM_, NT_, false);                                                  \
    } while (0)
#define OASIS_STS_SMALL(QT_)                         \
    do {                                             \
        if (nt == 512) {                             \
            if (C <= 8) OASIS_STS(QT_, 8, 512);      \
            else OASIS_STS(QT_, 16, 512);            \
        } else if (C <= 4) OASIS_STS(QT_, 4, 256);   \
        else OASIS_STS(QT_, 8, 256);                 \
    } while (0)
#define OASIS_STS_LARGE(QT_)                  \
    do {                                      \
        if (C <= 4) OASIS_STS(QT_, 4, 256);   \
        else if (C <= 8) OASIS_STS(QT_, 8, 256); \
        else if (C <= 16) OASIS_STS(QT_, 16, 256); \
        else OASIS_STS(QT_, 32, 256);         \
    } while (0)
    if (QT == 1) OASIS_STS_SMALL(1);
    else if (QT == 2) OASIS_STS_SMALL(2);
    else if (QT == 3) OASIS_STS_LARGE(3);
    else OASIS_STS_LARGE(4);
#undef OASIS_STS_LARGE
#undef OASIS_STS_SMALL
#undef OASIS_STS
#undef OASIS_STS_X
    return hipGetLastError();
}

hipError_t launch_evict(const Dims &D, const int32_t *blocks, const int32_t *counts,
                        int max_per_unit, int32_t *slot_block, int32_t *block_slot,
                        hipStream_t st) {
    OASIS_LAUNCH(evict_kernel, dim3((unsigned)D.units()), dim3(64), 0, st, blocks, counts,
                       max_per_unit, slot_block, block_slot, D.S, D.NBmax);
    return hipGetLastError();
}

hipError_t launch_evict_attended(const Dims &D, const double *draws, double fraction,
                                const int32_t *att_block, const int32_t *counts,
                                int32_t *slot_block, int32_t *block_slot, hipStream_t st) {
    if (D.K > 1024) return hipErrorInvalidValue;
    OASIS_LAUNCH(evict_attended_kernel, dim3((unsigned)D.units()), dim3(256), 0, st, draws,
                 fraction, att_block, counts, slot_block, block_slot, D.K, D.S, D.NBmax);
    return hipGetLastError();
}

hipError_t launch_rebuild_block_slot(const Dims &D, const int32_t *slot_block,
                                     int32_t *block_slot, hipStream_t st) {
    // one workgroup per unit so the clear is ordered before the fill
    OASIS_LAUNCH(rebuild_block_slot_kernel, dim3(1, (unsigned)D.units()), dim3(256), 0, st,
                       slot_block, block_slot, D.S, D.NBmax);
    return hipGetLastError();
}

}  // namespace oasis
