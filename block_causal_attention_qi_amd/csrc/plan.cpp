// Host side of libqi: wave validation, block offsets, row tiles, XCD-aware launch
// schedules, prefix-cache layout, tile classification and pair counts.  No HIP calls.
//
// The block structure follows the pages: a request is a text-instruction block, then its
// reference-image blocks in the order given, then the image-latent block (ThakiCloud blog
// "Qwen-Image-2.1 vLLM-Omni day 0", section "Serving architecture: the cross-step prefix
// KV cache"; vLLM recipe "Qwen/Qwen-Image-2.1", section "Offline inference" for the
// reference order).  A wave is a set of requests at the same denoising phase (recipe,
// section "Online serving").
#include <algorithm>
#include <cmath>
#include <map>
#include <tuple>
#include <cstring>
#include <new>
#include <numeric>

#include "qi_internal.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Rows of a call for one request: list of (first row, row count) blocks, and key count.
void call_blocks(const qi_req_host &r, int call, std::vector<std::pair<int, int>> &blocks,
                 int &nkeys) {
  const int nb = (int)r.bl.size();
  int b0 = 0, b1 = nb;
  if (call == QI_CALL_PREFIX) {
    b1 = nb - 1;
    nkeys = r.lp;
  } else if (call == QI_CALL_DENOISE) {
    b0 = nb - 1;
    nkeys = r.n;
  } else {
    nkeys = r.n;
  }
  blocks.clear();
  for (int b = b0; b < b1; ++b) blocks.emplace_back((int)r.off[b], r.bl[b]);
}

// Rows of a row tile [r0, r0 + nr) all lie in one block b; they see keys [0, off[b+1]).
int visible_end(const qi_req_host &r, int row) {
  for (size_t b = 0; b + 1 < r.off.size(); ++b)
    if (row < r.off[b + 1]) return (int)r.off[b + 1];
  return r.n;
}

struct Unit {           // all row tiles of one (request, head): they read the same K/V
  int req, head;
  int64_t cost;         // sum of item costs
  std::vector<int> tiles;
};

// Cost of one (row tile, head) item: key tiles visited x 128-row blocks.
int64_t item_cost(const qi_tile &t) {
  return (int64_t)((t.k1 - t.k0 + QI_KERNEL_BN - 1) / QI_KERNEL_BN) * ((t.nrows + 127) / 128);
}

// Deal the (tile, head) items of a call to the XCDs and order them for launch.
//  1. Units (request, head) go to XCDs longest-processing-time first, so the row tiles
//     that stream one head's K/V run on one XCD and share its L2.  When whole units
//     cannot balance the XCDs (12 equal heads on 8 XCDs leave four XCDs with twice the
//     work of the others), units are cut into runs of 32, 16, ... consecutive row tiles,
//     keeping the cut that shortens the estimated launch (per XCD, the larger of its work
//     over its workgroup slots and its longest item) by more than 2%, the first that comes
//     within 2% of the lower bound; a head whose runs land on two XCDs is read into both
//     L2s, a small cost next to an idle XCD.
//  2. Per XCD the items are list-scheduled (longest first) on the XCD's workgroup slots.
//     An item of more than 128 rows whose whole placement would end later than both the
//     current makespan and the load-balance bound is split into its two 128-row halves
//     (appended to the tile table); the kernel runs such halves with the key tiles split
//     over its two wavefront groups, so no slot sits idle at the end of the launch.
//  3. The per-XCD lists, longest item first, are interleaved in launch order (workgroup i
//     runs on XCD i % 8).
void build_schedule(const qi_plan &p, std::vector<qi_tile> &tiles,
                    const std::vector<std::pair<int, int>> &items_in, int slots_per_xcd,
                    bool may_split, bool chunked, std::vector<int32_t> &sched) {
  using Bins = std::vector<std::vector<std::pair<int, int>>>;   // (tile, head) per XCD
  // units of at most run_tiles row tiles, dealt to the XCDs longest first; returns the
  // estimated launch length in item-cost units
  auto deal = [&](int run_tiles, Bins &bins, std::vector<int64_t> &load) {
    std::vector<Unit> units;
    std::map<std::tuple<int, int, int, int>, int> unit_of;
    std::map<std::tuple<int, int, int>, int> run_len;
    for (auto [t, h] : items_in) {
      // a unit shares one stream of K/V: (request, head), or with key chunks (request,
      // head, chunk); cut into runs of consecutive row tiles
      const int k0 = chunked ? tiles[t].k0 : 0;
      const int run = run_len[{tiles[t].req, h, k0}]++ / run_tiles;
      const auto key = std::make_tuple(tiles[t].req, h, k0, run);
      auto it = unit_of.find(key);
      if (it == unit_of.end()) {
        it = unit_of.emplace(key, (int)units.size()).first;
        units.push_back(Unit{tiles[t].req, h, 0, {}});
      }
      units[it->second].tiles.push_back(t);
      units[it->second].cost += item_cost(tiles[t]);
    }
    for (Unit &u : units)
      std::stable_sort(u.tiles.begin(), u.tiles.end(), [&](int a, int b) {
        return item_cost(tiles[a]) > item_cost(tiles[b]);   // longest row tiles first
      });
    std::stable_sort(units.begin(), units.end(),
                     [](const Unit &a, const Unit &b) { return a.cost > b.cost; });
    bins.assign(QI_NUM_XCD, {});
    load.assign(QI_NUM_XCD, 0);
    std::vector<int64_t> longest(QI_NUM_XCD, 0);
    for (const Unit &u : units) {
      int best = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      load[best] += u.cost;
      for (int t : u.tiles) {
        bins[best].push_back({t, u.head});
        longest[best] = std::max(longest[best], item_cost(tiles[t]));
      }
    }
    int64_t est = 0;
    for (int x = 0; x < QI_NUM_XCD; ++x)
      est = std::max(est, std::max((load[x] + slots_per_xcd - 1) / slots_per_xcd, longest[x]));
    return est;
  };
  // a head shard's key chunks: runs of at most 8 row tiles (too few (request, head) pairs
  // to spread over the XCDs); otherwise whole units unless they leave the XCDs unbalanced
  Bins bins;
  std::vector<int64_t> load;
  int64_t est = deal(chunked ? 8 : (1 << 30), bins, load);
  if (!chunked) {
    int64_t total = 0, longest = 0;
    for (int64_t l : load) total += l;
    for (auto [t, h] : items_in) longest = std::max(longest, item_cost(tiles[t]));
    const int64_t slots = (int64_t)QI_NUM_XCD * slots_per_xcd;
    const int64_t bound = std::max((total + slots - 1) / slots, longest);
    for (int run_tiles = 32; run_tiles >= 1 && est * 50 > bound * 51; run_tiles /= 2) {
      Bins b2;
      std::vector<int64_t> l2;
      const int64_t e2 = deal(run_tiles, b2, l2);
      if (e2 * 51 < est * 50) {   // more than 2% shorter
        est = e2;
        bins.swap(b2);
        load.swap(l2);
      }
    }
  }
  std::vector<std::vector<int32_t>> lists(QI_NUM_XCD);
  for (int x = 0; x < QI_NUM_XCD; ++x) {
    auto &items = bins[x];
    std::stable_sort(items.begin(), items.end(), [&](const auto &a, const auto &b) {
      return item_cost(tiles[a.first]) > item_cost(tiles[b.first]);
    });
    const int64_t bound = (load[x] + slots_per_xcd - 1) / slots_per_xcd;
    std::vector<int64_t> slot(slots_per_xcd, 0);
    int64_t makespan = 0;
    std::vector<std::pair<int64_t, int32_t>> placed;   // (cost, item code)
    auto least = [&]() { return (int)(std::min_element(slot.begin(), slot.end()) - slot.begin()); };
    for (auto [t, h] : items) {
      const int64_t c = item_cost(tiles[t]);
      const int s0 = least();
      bool split = false;
      if (may_split && tiles[t].nrows > 128 && slot[s0] + c > std::max(makespan, bound)) {
        const int64_t c1 = c / 2;   // both halves see the same keys
        std::vector<int64_t> trial = slot;
        int a = (int)(std::min_element(trial.begin(), trial.end()) - trial.begin());
        trial[a] += c1;
        int b = (int)(std::min_element(trial.begin(), trial.end()) - trial.begin());
        trial[b] += c1;
        split = std::max(trial[a], trial[b]) < slot[s0] + c;
      }
      if (!split) {
        slot[s0] += c;
        makespan = std::max(makespan, slot[s0]);
        placed.push_back({c, t * p.H + h});
      } else {
        // new entries for both halves: a tile entry is shared by every head's item
        qi_tile lo = tiles[t], hi = tiles[t];
        lo.nrows = 128;
        hi.q_tok += 128;
        hi.nrows = tiles[t].nrows - 128;
        const int t1 = (int)tiles.size();
        tiles.push_back(lo);
        tiles.push_back(hi);
        for (int half : {t1, t1 + 1}) {
          const int s = least();
          slot[s] += item_cost(tiles[half]);
          makespan = std::max(makespan, slot[s]);
          placed.push_back({item_cost(tiles[half]), half * p.H + h});
        }
      }
    }
    std::stable_sort(placed.begin(), placed.end(),
                     [](const auto &a, const auto &b) { return a.first > b.first; });
    for (auto &pc : placed) lists[x].push_back(pc.second);
  }
  size_t len = 0;
  for (auto &l : lists) len = std::max(len, l.size());
  sched.assign(len * QI_NUM_XCD, -1);
  for (size_t s2 = 0; s2 < len; ++s2)
    for (int x = 0; x < QI_NUM_XCD; ++x)
      if (s2 < lists[x].size()) sched[s2 * QI_NUM_XCD + x] = lists[x][s2];
}

void build_tiles(const qi_plan &p, int call, std::vector<qi_tile> &tiles) {
  tiles.clear();
  const int bm = p.bm[call];
  std::vector<std::pair<int, int>> blocks;
  for (int r = 0; r < p.n_req; ++r) {
    const qi_req_host &rq = p.req[r];
    int nkeys = 0;
    call_blocks(rq, call, blocks, nkeys);
    for (auto [start, len] : blocks) {
      for (int r0 = start; r0 < start + len; r0 += bm) {
        qi_tile t{};
        t.nrows = std::min(bm, start + len - r0);
        t.kend = std::min(visible_end(rq, r0), nkeys);
        t.k0 = 0;
        t.k1 = t.kend;
        t.part = -1;
        t.req = r;
        t.k_off = rq.k_off;
        t.v_off = rq.v_off;
        t.s_off = rq.s_off;
        if (call == QI_CALL_PREFIX) {
          t.q_tok = rq.pre_tok + r0;
          t.kv_tok = rq.pre_tok;
          t.lp = 0;
        } else if (call == QI_CALL_DENOISE) {
          t.q_tok = rq.img_tok + (r0 - rq.lp);
          t.kv_tok = rq.img_tok;
          t.lp = rq.lp;
        } else {
          t.q_tok = rq.all_tok + r0;
          t.kv_tok = rq.all_tok;
          t.lp = 0;
        }
        tiles.push_back(t);
      }
    }
  }
}

// Key tiles a row tile visits without a key split.
int key_tiles(const qi_tile &t) { return (t.kend + QI_KERNEL_BN - 1) / QI_KERNEL_BN; }

// Key split.  When the prefix or the denoising call has fewer (row tile, head) items than
// compute units (a head-sharded deployment: three heads of 24 per GPU), much of the chip
// would idle, so every row tile's keys are cut into chunks of ct key tiles, each its own
// workgroup, and the chunks' partial softmax states are merged afterwards.  ct minimises
// an estimate of the call's time in key-tile units: rounds of one workgroup per CU times
// (the longest chunk plus a workgroup's fixed cost), plus the merge's traffic per partial
// slot; the split is taken only when that beats the whole row tiles by more than 5%.
// 0: no split.  Each of the two calls picks its own ct; the full call runs every row in
// the chunks of the call that owns the row, so reuse stays bit-identical.
constexpr double kWgFixedTiles = 2.0;     // prologue (Q and first tiles) and epilogue
constexpr double kMergeSlotTiles = 0.03;  // a slot's partial state written and read back
double split_cost(const std::vector<qi_tile> &den, int H, int ct) {
  int64_t wgs = 0;
  int longest = 0;
  for (const qi_tile &t : den) {
    const int n = key_tiles(t);
    wgs += (int64_t)H * (ct > 0 ? (n + ct - 1) / ct : 1);
    longest = std::max(longest, ct > 0 ? std::min(ct, n) : n);
  }
  const double rounds = (double)((wgs + QI_NUM_CUS - 1) / QI_NUM_CUS);
  return rounds * (longest + kWgFixedTiles) + (ct > 0 ? wgs * kMergeSlotTiles : 0.0);
}
int choose_chunk_tiles(const std::vector<qi_tile> &den, int H) {
  if (den.empty() || (int64_t)den.size() * H >= QI_NUM_CUS) return 0;
  int max_t = 0;
  for (const qi_tile &t : den) max_t = std::max(max_t, key_tiles(t));
  int best = 0;
  double best_cost = 0.95 * split_cost(den, H, 0);
  for (int ct = QI_SPLIT_MIN_TILES; ct < max_t; ++ct) {
    const double c = split_cost(den, H, ct);
    if (c < best_cost) {
      best_cost = c;
      best = ct;
    }
  }
  return best;
}

// Cut the row tiles of one call into key chunks of ct tiles: a row tile of more than ct
// key tiles becomes nchunks tiles (chunk s: keys [s ct BN, min((s+1) ct BN, kend)),
// partial slots part0 + s H + head) and one merge entry; the others stay whole.  Partial
// slots are numbered from 0 per call.
void split_keys(int ct, int H, std::vector<qi_tile> &tiles, std::vector<qi_merge> &merges,
                std::vector<int> &merge_req, int64_t &slots) {
  merges.clear();
  merge_req.clear();
  slots = 0;
  if (ct <= 0) return;
  std::vector<qi_tile> out;
  for (const qi_tile &t : tiles) {
    const int nt = key_tiles(t);
    if (nt <= ct) {
      out.push_back(t);
      continue;
    }
    const int nch = (nt + ct - 1) / ct;
    merges.push_back(qi_merge{t.q_tok, t.nrows, nch, (int32_t)slots});
    merge_req.push_back(t.req);
    for (int c = 0; c < nch; ++c) {
      qi_tile u = t;
      u.k0 = c * ct * QI_KERNEL_BN;
      u.k1 = std::min((c + 1) * ct * QI_KERNEL_BN, t.kend);
      u.part = (int32_t)(slots + (int64_t)c * H);
      u.pad = c;   // chunk index (host bookkeeping)
      out.push_back(u);
    }
    slots += (int64_t)nch * H;
  }
  tiles.swap(out);
}

template <typename T>
void put(std::vector<uint8_t> &img, size_t off, const std::vector<T> &v) {
  if (!v.empty()) std::memcpy(img.data() + off, v.data(), v.size() * sizeof(T));
}

}  // namespace

extern "C" {

const char *qi_status_string(qi_status st) {
  switch (st) {
    case QI_OK: return "ok";
    case QI_ERR_INVALID_ARG: return "invalid argument";
    case QI_ERR_UNSUPPORTED: return "unsupported configuration";
    case QI_ERR_STATE: return "call out of order (workspace not uploaded or cache never built)";
    case QI_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case QI_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

qi_status qi_plan_create(const qi_wave_desc *d, qi_plan **out) {
  if (!out) return QI_ERR_INVALID_ARG;
  *out = nullptr;
  if (!d || !d->n_refs || !d->block_len) return QI_ERR_INVALID_ARG;
  if (d->n_requests < 1 || d->n_requests > QI_MAX_REQUESTS) return QI_ERR_INVALID_ARG;
  if (d->n_heads < 1 || d->n_heads > QI_MAX_HEADS) return QI_ERR_INVALID_ARG;
  if (d->kv_dtype != QI_KV_BF16 && d->kv_dtype != QI_KV_FP8_E4M3 && d->kv_dtype != QI_KV_FP8_V)
    return QI_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return QI_ERR_UNSUPPORTED;

  qi_plan *p = new (std::nothrow) qi_plan();
  if (!p) return QI_ERR_INVALID_ARG;
  p->n_req = d->n_requests;
  p->H = d->n_heads;
  p->D = d->head_dim;
  p->kv = d->kv_dtype;
  const int ebk = qi_cache_elem_bytes(p->kv, 0), ebv = qi_cache_elem_bytes(p->kv, 1);

  // requests, block offsets, packed token bases, cache layout
  size_t pos = 0, cache_end = 0;
  for (int r = 0; r < p->n_req; ++r) {
    const int nr = d->n_refs[r];
    if (nr < 0 || nr > QI_MAX_REFS) { delete p; return QI_ERR_INVALID_ARG; }
    qi_req_host rq;
    int64_t tot = 0;
    rq.off.push_back(0);
    for (int b = 0; b < nr + 2; ++b) {
      const int32_t len = d->block_len[pos + b];
      if (len <= 0) { delete p; return QI_ERR_INVALID_ARG; }
      rq.bl.push_back(len);
      tot += len;
      if (tot >= (int64_t(1) << 24)) { delete p; return QI_ERR_INVALID_ARG; }
      rq.off.push_back(tot);
    }
    pos += nr + 2;
    rq.n = (int32_t)tot;
    rq.nimg = rq.bl.back();
    rq.lp = rq.n - rq.nimg;
    rq.pre_tok = (int32_t)p->tot_pre;
    rq.img_tok = (int32_t)p->tot_img;
    rq.all_tok = (int32_t)p->tot_all;
    p->tot_pre += rq.lp;
    p->tot_img += rq.nimg;
    p->tot_all += rq.n;
    const size_t elems = (size_t)p->H * rq.lp * p->D;
    rq.k_off = (int64_t)align_up(cache_end);
    rq.v_off = (int64_t)align_up(rq.k_off + elems * ebk);
    rq.end = rq.v_off + (int64_t)(elems * ebv);
    if (p->kv != QI_KV_BF16) {
      rq.s_off = (int64_t)align_up(rq.end);
      rq.end = rq.s_off + 2 * 4 * p->H;
    }
    cache_end = (size_t)rq.end;
    p->req.push_back(std::move(rq));
  }
  // every packed tensor must stay addressable with 32-bit element indices
  if (p->tot_all * p->H * p->D >= (int64_t(1) << 31)) { delete p; return QI_ERR_INVALID_ARG; }
  p->cache_bytes = align_up(cache_end);

  // useful pairs: rows of block b see keys [0, off[b+1])
  for (const qi_req_host &rq : p->req) {
    const int nb = (int)rq.bl.size();
    for (int b = 0; b < nb; ++b) {
      const int64_t pr = (int64_t)rq.bl[b] * rq.off[b + 1];
      p->pairs[QI_CALL_FULL] += pr;
      if (b < nb - 1) p->pairs[QI_CALL_PREFIX] += pr;
      else p->pairs[QI_CALL_DENOISE] += pr;
    }
  }

  // device tables: per-request records, tiles and schedules of the three calls, partials
  std::vector<qi_req_dev> reqs(p->n_req);
  size_t nparts = 0;
  for (int r = 0; r < p->n_req; ++r) {
    const qi_req_host &rq = p->req[r];
    qi_req_dev &e = reqs[r];
    e.pre_tok = rq.pre_tok;
    e.lp = rq.lp;
    e.n_chunks = (rq.lp + QI_CACHE_CHUNK - 1) / QI_CACHE_CHUNK;
    e.part_idx = (int32_t)nparts;
    e.k_off = rq.k_off;
    e.v_off = rq.v_off;
    e.s_off = rq.s_off;
    e.pad = 0;
    nparts += (size_t)e.n_chunks * 2 * p->H;
    p->max_chunks = std::max(p->max_chunks, e.n_chunks);
  }
  std::vector<qi_tile> tiles[3];
  std::vector<int32_t> sched[3];
  std::vector<qi_merge> merges[3];
  std::vector<int> merge_req[3];
  int64_t slots[3] = {0, 0, 0};
  // prefix and denoising calls: row tiles per block, balanced (and split) per call.  The
  // full call reuses exactly their decomposition, (row tile, head) by (row tile, head),
  // so every row runs the same kernel path over the same key tiles in every call and the
  // results agree bit for bit (reuse is exact).
  for (int c : {QI_CALL_PREFIX, QI_CALL_DENOISE}) {
    p->bm[c] = QI_ROWS;
    build_tiles(*p, c, tiles[c]);
  }
  for (int c : {QI_CALL_PREFIX, QI_CALL_DENOISE}) {
    p->kchunk_tiles[c] = choose_chunk_tiles(tiles[c], p->H);
    split_keys(p->kchunk_tiles[c], p->H, tiles[c], merges[c], merge_req[c], slots[c]);
    std::vector<std::pair<int, int>> items;
    for (int t = 0; t < (int)tiles[c].size(); ++t)
      for (int h = 0; h < p->H; ++h) items.push_back({t, h});
    // the kernel runs one 8-wavefront workgroup per CU; key-split plans keep row tiles
    // whole (their chunks already fill the chip)
    build_schedule(*p, tiles[c], items, QI_CUS_PER_XCD, p->kchunk_tiles[c] == 0,
                   p->kchunk_tiles[c] > 0, sched[c]);
  }
  {
    p->bm[QI_CALL_FULL] = QI_ROWS;
    std::vector<std::pair<int, int>> items;
    std::vector<qi_tile> &ft = tiles[QI_CALL_FULL];
    for (int c : {QI_CALL_PREFIX, QI_CALL_DENOISE}) {
      // the source call's merge groups get slots of their own in the full call
      std::vector<int64_t> base_of(merges[c].size());
      std::vector<int> group_of_part;   // source slot base -> merge group
      for (size_t m = 0; m < merges[c].size(); ++m) {
        const qi_merge &e = merges[c][m];
        const qi_req_host &rq = p->req[merge_req[c][m]];
        const int r0 = c == QI_CALL_PREFIX ? e.q_tok - rq.pre_tok : e.q_tok - rq.img_tok + rq.lp;
        base_of[m] = slots[QI_CALL_FULL];
        merges[QI_CALL_FULL].push_back(
            qi_merge{rq.all_tok + r0, e.nrows, e.nchunks, (int32_t)slots[QI_CALL_FULL]});
        merge_req[QI_CALL_FULL].push_back(merge_req[c][m]);
        slots[QI_CALL_FULL] += (int64_t)e.nchunks * p->H;
        if ((int)group_of_part.size() <= e.part0) group_of_part.resize(e.part0 + 1, -1);
        group_of_part[e.part0] = (int)m;
      }
      std::vector<int> map(tiles[c].size(), -1);
      for (int32_t code : sched[c]) {
        if (code < 0) continue;
        const int t = code / p->H, h = code % p->H;
        if (map[t] < 0) {
          const qi_tile &src = tiles[c][t];
          const qi_req_host &rq = p->req[src.req];
          const int r0 = c == QI_CALL_PREFIX ? src.q_tok - rq.pre_tok
                                             : src.q_tok - rq.img_tok + rq.lp;
          qi_tile f = src;
          f.q_tok = rq.all_tok + r0;
          f.kv_tok = rq.all_tok;
          f.lp = 0;
          if (src.part >= 0) {
            const int g = group_of_part[src.part - src.pad * p->H];
            f.part = (int32_t)(base_of[g] + (int64_t)src.pad * p->H);
          }
          map[t] = (int)ft.size();
          ft.push_back(f);
        }
        items.push_back({map[t], h});
      }
    }
    build_schedule(*p, ft, items, QI_CUS_PER_XCD, false,
                   p->kchunk_tiles[QI_CALL_PREFIX] > 0 || p->kchunk_tiles[QI_CALL_DENOISE] > 0,
                   sched[QI_CALL_FULL]);
  }
  p->kpart_slots = std::max({slots[0], slots[1], slots[2]});
  size_t off = 0;
  p->reqs_off = off;
  off = align_up(off + reqs.size() * sizeof(qi_req_dev));
  for (int c = 0; c < 3; ++c) {
    p->n_tiles[c] = (int32_t)tiles[c].size();
    p->sched_len[c] = (int32_t)sched[c].size();
    p->tiles_off[c] = off;
    off = align_up(off + tiles[c].size() * sizeof(qi_tile));
    p->sched_off[c] = off;
    off = align_up(off + sched[c].size() * sizeof(int32_t));
    p->n_merge[c] = (int32_t)merges[c].size();
    p->merge_off[c] = off;
    off = align_up(off + merges[c].size() * sizeof(qi_merge));
  }
  p->part_off = off;
  p->part_floats = p->kv != QI_KV_BF16 ? nparts : 0;
  off = align_up(off + p->part_floats * sizeof(float));
  p->kpart_off = off;
  off = align_up(off + (size_t)p->kpart_slots * QI_PART_SLOT_FLOATS(p->D) * sizeof(float));
  p->ws_bytes = off;
  p->ws_image.assign(p->part_off, 0);
  put(p->ws_image, p->reqs_off, reqs);
  for (int c = 0; c < 3; ++c) {
    put(p->ws_image, p->tiles_off[c], tiles[c]);
    put(p->ws_image, p->sched_off[c], sched[c]);
    put(p->ws_image, p->merge_off[c], merges[c]);
  }
  *out = p;
  return QI_OK;
}

void qi_plan_destroy(qi_plan *p) { delete p; }

qi_status qi_plan_sizes(const qi_plan *p, size_t *cache_bytes, size_t *workspace_bytes) {
  if (!p) return QI_ERR_INVALID_ARG;
  if (cache_bytes) *cache_bytes = p->cache_bytes;
  if (workspace_bytes) *workspace_bytes = p->ws_bytes;
  return QI_OK;
}

qi_status qi_plan_kernel_tile(const qi_plan *p, int32_t call, int32_t *bm, int32_t *bn) {
  if (!p || !bm || !bn || call < 0 || call > 2) return QI_ERR_INVALID_ARG;
  *bm = p->bm[call];
  *bn = QI_KERNEL_BN;
  return QI_OK;
}

qi_status qi_plan_tile_map(const qi_plan *p, int32_t call, int32_t bm, int32_t bn,
                           uint8_t *host_out, size_t n, size_t *n_needed) {
  if (!p || call < 0 || call > 2 || bm < 1 || bn < 1) return QI_ERR_INVALID_ARG;
  std::vector<std::pair<int, int>> blocks;
  size_t need = 0;
  for (const qi_req_host &rq : p->req) {
    int nkeys = 0;
    call_blocks(rq, call, blocks, nkeys);
    size_t rows = 0;
    for (auto [start, len] : blocks) rows += (len + bm - 1) / bm;
    need += rows * (size_t)((nkeys + bn - 1) / bn);
  }
  if (n_needed) *n_needed = need;
  if (!host_out || n < need) return QI_ERR_BUFFER_TOO_SMALL;
  size_t w = 0;
  for (const qi_req_host &rq : p->req) {
    int nkeys = 0;
    call_blocks(rq, call, blocks, nkeys);
    const int nkt = (nkeys + bn - 1) / bn;
    for (auto [start, len] : blocks) {
      const int vis = std::min(visible_end(rq, start), nkeys);
      for (int r0 = start; r0 < start + len; r0 += bm) {
        for (int j = 0; j < nkt; ++j) {
          const int k0 = j * bn, k1 = std::min(nkeys, (j + 1) * bn);
          host_out[w++] = k1 <= vis ? 2 : (k0 >= vis ? 0 : 1);
        }
      }
    }
  }
  return QI_OK;
}

qi_status qi_plan_launch_items(const qi_plan *p, int32_t call, int32_t *host_out, size_t n,
                               size_t *n_needed) {
  if (!p || call < 0 || call > 2) return QI_ERR_INVALID_ARG;
  const size_t len = (size_t)p->sched_len[call];
  if (n_needed) *n_needed = QI_LAUNCH_ITEM_FIELDS * len;
  if (!host_out || n < QI_LAUNCH_ITEM_FIELDS * len) return QI_ERR_BUFFER_TOO_SMALL;
  const int32_t *sched = reinterpret_cast<const int32_t *>(p->ws_image.data() + p->sched_off[call]);
  const qi_tile *tiles = reinterpret_cast<const qi_tile *>(p->ws_image.data() + p->tiles_off[call]);
  for (size_t i = 0; i < len; ++i) {
    int32_t *e = host_out + QI_LAUNCH_ITEM_FIELDS * i;
    const int32_t code = sched[i];
    if (code < 0) {
      for (int f = 0; f < QI_LAUNCH_ITEM_FIELDS; ++f) e[f] = -1;
      continue;
    }
    const qi_tile &t = tiles[code / p->H];
    const qi_req_host &rq = p->req[t.req];
    const int32_t base = call == QI_CALL_PREFIX ? rq.pre_tok
                         : call == QI_CALL_DENOISE ? rq.img_tok - rq.lp : rq.all_tok;
    e[0] = t.req;
    e[1] = code % p->H;
    e[2] = t.q_tok - base;
    e[3] = t.nrows;
    e[4] = t.k0;
    e[5] = t.k1;
  }
  return QI_OK;
}

qi_status qi_plan_cache_offset(const qi_plan *p, int32_t req, int32_t kv, int32_t head,
                               int32_t tok, size_t *byte_off) {
  if (!p || !byte_off || req < 0 || req >= p->n_req || kv < 0 || kv > 2) return QI_ERR_INVALID_ARG;
  const qi_req_host &rq = p->req[req];
  if (kv == 2) {
    if (p->kv == QI_KV_BF16) return QI_ERR_INVALID_ARG;
    *byte_off = (size_t)rq.s_off;
    return QI_OK;
  }
  if (head < 0 || head >= p->H || tok < 0 || tok >= rq.lp) return QI_ERR_INVALID_ARG;
  const size_t eb = qi_cache_elem_bytes(p->kv, kv);
  *byte_off = (size_t)(kv == 0 ? rq.k_off : rq.v_off) + ((size_t)head * rq.lp + tok) * p->D * eb;
  return QI_OK;
}

qi_status qi_plan_pairs(const qi_plan *p, int32_t call, int64_t *pairs) {
  if (!p || !pairs || call < 0 || call > 2) return QI_ERR_INVALID_ARG;
  *pairs = p->pairs[call];
  return QI_OK;
}

qi_status qi_plan_tokens(const qi_plan *p, int64_t *pre, int64_t *img, int64_t *all) {
  if (!p) return QI_ERR_INVALID_ARG;
  if (pre) *pre = p->tot_pre;
  if (img) *img = p->tot_img;
  if (all) *all = p->tot_all;
  return QI_OK;
}

}  // extern "C"
