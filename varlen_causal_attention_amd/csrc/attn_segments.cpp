// Document-causal segment layout on the host ("fa4" page: module overview of
// document-causal attention and the _varlen_segments / _varlen_layout entries;
// "gemma4_moe cp_attention" page: ring segments pair a document's queries of
// one shard with its keys in one KV chunk, cu_q[i] pairing cu_k[i]).
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "attn_error.hpp"

namespace {

struct Run {
  int begin, end, id;  // positions [begin, end) of one row carrying document id
};

// Maximal runs of equal id inside positions [a, b) of one row.
std::vector<Run> runs_of(const int32_t* ids, int a, int b) {
  std::vector<Run> out;
  int p = a;
  while (p < b) {
    int e = p + 1;
    while (e < b && ids[e] == ids[p]) ++e;
    out.push_back(Run{p, e, ids[p]});
    p = e;
  }
  return out;
}

}  // namespace

namespace {

// Per-segment query and key lengths of the layout (the attn_doc_segments
// rules); ATTN_OK or ATTN_E_INVALID with the error text set.
int build_segments(const int32_t* doc_ids, int B, int S, int q_start, int q_len, int k_start,
                   int k_len, int mode, std::vector<int32_t>& sq, std::vector<int32_t>& sk) {
  if (!doc_ids || B < 0 || S < 0 || q_len < 0 || k_len < 0 || q_start < 0 ||
      k_start < 0 || q_start + q_len > S || k_start + k_len > S || (mode != 0 && mode != 1)) {
    vca::set_last_error("doc layout: invalid arguments");
    return ATTN_E_INVALID;
  }
  const int q_end = q_start + q_len, k_end = k_start + k_len;
  if (mode == 0 && !(k_start <= q_start && q_end <= k_end)) {
    vca::set_last_error("doc layout: causal mode needs the key range to cover the query range");
    return ATTN_E_INVALID;
  }
  if (mode == 1 && k_end > q_start) {
    vca::set_last_error("doc layout: cross mode needs every key before every query");
    return ATTN_E_INVALID;
  }
  for (int b = 0; b < B; ++b) {
    const int32_t* ids = doc_ids + (size_t)b * S;
    if (mode == 0) {
      // split every run of the key range at the query-shard end; a piece that
      // ends inside the shard carries its queries (the part inside the shard)
      // and all of its keys; other pieces only keys.
      for (const Run& r0 : runs_of(ids, k_start, k_end)) {
        Run pieces[2] = {r0, r0};
        int np = 1;
        if (r0.begin < q_end && q_end < r0.end) {
          pieces[0].end = q_end;
          pieces[1].begin = q_end;
          np = 2;
        }
        for (int i = 0; i < np; ++i) {
          const Run& r = pieces[i];
          const int qa = r.begin > q_start ? r.begin : q_start;
          const int qb = r.end < q_end ? r.end : q_end;
          const int nq = qb > qa ? qb - qa : 0;
          const int nk = r.end - r.begin;
          if (r.id == 0 && nq > 0) {
            // padding: queries attend nothing, keys are seen by nobody
            sq.push_back(nq);
            sk.push_back(0);
            sq.push_back(0);
            sk.push_back(nk);
          } else {
            sq.push_back(r.id == 0 ? 0 : nq);
            sk.push_back(nk);
          }
        }
      }
    } else {
      // cross chunk: merge the runs of the key range and of the query range in
      // position order; a document present in both pairs up, others stand alone.
      std::vector<Run> kr = runs_of(ids, k_start, k_end);
      std::vector<Run> qr = runs_of(ids, q_start, q_end);
      size_t i = 0, j = 0;
      while (i < kr.size() || j < qr.size()) {
        if (i < kr.size() && j < qr.size() && kr[i].id == qr[j].id && kr[i].id != 0) {
          sq.push_back(qr[j].end - qr[j].begin);
          sk.push_back(kr[i].end - kr[i].begin);
          ++i;
          ++j;
        } else if (i < kr.size() && (j >= qr.size() || kr[i].begin < qr[j].begin)) {
          sq.push_back(0);
          sk.push_back(kr[i].end - kr[i].begin);
          ++i;
        } else {
          sq.push_back(qr[j].end - qr[j].begin);
          sk.push_back(0);
          ++j;
        }
      }
    }
  }
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_doc_segments(const int32_t* doc_ids, int B, int S, int q_start, int q_len,
                                 int k_start, int k_len, int mode, int32_t* seg_q, int32_t* seg_k,
                                 int max_segments, int* num_segments) {
  vca::set_last_error("");
  if (!num_segments) {
    vca::set_last_error("attn_doc_segments: invalid arguments");
    return ATTN_E_INVALID;
  }
  std::vector<int32_t> sq, sk;
  const int st = build_segments(doc_ids, B, S, q_start, q_len, k_start, k_len, mode, sq, sk);
  if (st != ATTN_OK) return st;
  *num_segments = (int)sq.size();
  if ((int)sq.size() > max_segments || !seg_q || !seg_k) {
    vca::set_last_error("attn_doc_segments: max_segments too small, " + std::to_string(sq.size()) +
                        " needed");
    return ATTN_E_INVALID;
  }
  for (size_t i = 0; i < sq.size(); ++i) {
    seg_q[i] = sq[i];
    seg_k[i] = sk[i];
  }
  return ATTN_OK;
}

// The same layout as cumulative offsets, ready for the varlen calls:
// cu_q[0] = cu_k[0] = 0 and cu_x[s + 1] = cu_x[s] + length of segment s.
extern "C" int attn_doc_cu_seqlens(const int32_t* doc_ids, int B, int S, int q_start, int q_len,
                                   int k_start, int k_len, int mode, int32_t* cu_q, int32_t* cu_k,
                                   int max_segments, int* num_segments, int* max_q, int* max_k) {
  vca::set_last_error("");
  if (!num_segments || !max_q || !max_k) {
    vca::set_last_error("attn_doc_cu_seqlens: invalid arguments");
    return ATTN_E_INVALID;
  }
  std::vector<int32_t> sq, sk;
  const int st = build_segments(doc_ids, B, S, q_start, q_len, k_start, k_len, mode, sq, sk);
  if (st != ATTN_OK) return st;
  *num_segments = (int)sq.size();
  if ((int)sq.size() > max_segments || !cu_q || !cu_k) {
    vca::set_last_error("attn_doc_cu_seqlens: max_segments too small, " +
                        std::to_string(sq.size()) + " needed");
    return ATTN_E_INVALID;
  }
  int mq = 0, mk = 0;
  cu_q[0] = cu_k[0] = 0;
  for (size_t i = 0; i < sq.size(); ++i) {
    cu_q[i + 1] = cu_q[i] + sq[i];
    cu_k[i + 1] = cu_k[i] + sk[i];
    mq = sq[i] > mq ? sq[i] : mq;
    mk = sk[i] > mk ? sk[i] : mk;
  }
  *max_q = mq;
  *max_k = mk;
  return ATTN_OK;
}

// Dense routing of one ring chunk ("gemma4_moe cp_attention" page: the
// dense-routing flags of the packed ring segments and the per-chunk dense
// eligibility entry; the single-document row predicates).
namespace {

// Positions [a, b) of one row hold one document id d > 0, then optionally
// padding (id 0) to b. Returns d, 0 when [a, b) is all padding, -1 otherwise.
int single_doc_prefix(const int32_t* ids, int a, int b) {
  if (a >= b || ids[a] == 0) {
    for (int p = a; p < b; ++p)
      if (ids[p] != 0) return -1;
    return 0;
  }
  const int d = ids[a];
  int p = a;
  while (p < b && ids[p] == d) ++p;
  while (p < b && ids[p] == 0) ++p;
  return p == b ? d : -1;
}

}  // namespace

extern "C" int attn_dense_route(const int32_t* doc_ids, int B, int S, int q_start, int q_len,
                                int k_start, int k_len, int mode, uint8_t* pad_rows,
                                int* eligible) {
  vca::set_last_error("");
  if (!doc_ids || !eligible || B < 0 || S < 0 || q_len < 0 || k_len < 0 || q_start < 0 ||
      k_start < 0 || q_start + q_len > S || k_start + k_len > S || (mode != 0 && mode != 1)) {
    vca::set_last_error("attn_dense_route: invalid arguments");
    return ATTN_E_INVALID;
  }
  const int q_end = q_start + q_len, k_end = k_start + k_len;
  if (mode == 0 && !(k_start <= q_start && q_end <= k_end)) {
    vca::set_last_error("attn_dense_route: causal mode needs the key range to cover the query range");
    return ATTN_E_INVALID;
  }
  if (mode == 1 && k_end > q_start) {
    vca::set_last_error("attn_dense_route: cross mode needs every key before every query");
    return ATTN_E_INVALID;
  }
  // Bottom-right causal alignment equals position causality only when the
  // key range ends where the query range ends.
  bool ok = mode == 1 || k_end == q_end;
  for (int b = 0; b < B && ok; ++b) {
    const int32_t* ids = doc_ids + (size_t)b * S;
    if (mode == 0) {
      // one document, padding only as a suffix: a query then sees exactly its
      // document's keys up to its own position; padding queries are zeroed
      ok = single_doc_prefix(ids, k_start, k_end) >= 0;
    } else {
      // keys: exactly one document, no padding; queries: that document, with
      // padding only as a suffix
      const int dk = single_doc_prefix(ids, k_start, k_end);
      bool kfull = dk > 0;
      for (int p = k_start; p < k_end && kfull; ++p) kfull = ids[p] == dk;
      const int dq = single_doc_prefix(ids, q_start, q_end);
      ok = kfull && (dq == dk || dq == 0);
    }
  }
  *eligible = ok ? 1 : 0;
  if (pad_rows)
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < q_len; ++i)
        pad_rows[(size_t)b * q_len + i] = doc_ids[(size_t)b * S + q_start + i] == 0 ? 1 : 0;
  return ATTN_OK;
}

// Packed ring segments with gather indices ("gemma4_moe cp_attention" page:
// the per-document varlen segments shared between a query shard and one KV
// chunk, returned as flat gather indices into B*S plus cu_seqlens). Every
// document id > 0 that occurs in both row b of the query shard and row b of
// the key chunk becomes one segment: its query positions (in order) and its
// key positions (in order), as flat indices b*Sq + p and b*Sk + p. Segments
// follow the rows, and within a row the order in which documents first occur
// among the queries. Documents in only one of the two, and padding, take no
// part, so only live tokens are gathered.
extern "C" int attn_ring_segments(const int32_t* q_ids, int Sq, const int32_t* k_ids, int Sk,
                                  int B, int32_t* q_index, int32_t* k_index, int32_t* cu_q,
                                  int32_t* cu_k, int max_segments, int* num_segments, int* Tq,
                                  int* Tk, int* max_q, int* max_k) {
  vca::set_last_error("");
  if (!q_ids || !k_ids || !num_segments || !Tq || !Tk || !max_q || !max_k || B < 0 || Sq < 0 ||
      Sk < 0 || (int64_t)B * Sq > INT32_MAX || (int64_t)B * Sk > INT32_MAX) {
    vca::set_last_error("attn_ring_segments: invalid arguments");
    return ATTN_E_INVALID;
  }
  std::vector<int32_t> qi, ki, cq{0}, ck{0};
  int mq = 0, mk = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t* qr = q_ids + (size_t)b * Sq;
    const int32_t* kr = k_ids + (size_t)b * Sk;
    std::vector<int32_t> order;  // documents in order of first occurrence among the queries
    for (int p = 0; p < Sq; ++p) {
      const int32_t d = qr[p];
      if (d <= 0) continue;
      bool seen = false;
      for (int32_t e : order) seen = seen || e == d;
      if (!seen) order.push_back(d);
    }
    for (int32_t d : order) {
      const size_t k0 = ki.size(), q0 = qi.size();
      for (int p = 0; p < Sk; ++p)
        if (kr[p] == d) ki.push_back((int32_t)((int64_t)b * Sk + p));
      if (ki.size() == k0) continue;  // not in the key chunk: no segment
      for (int p = 0; p < Sq; ++p)
        if (qr[p] == d) qi.push_back((int32_t)((int64_t)b * Sq + p));
      const int lq = (int)(qi.size() - q0), lk = (int)(ki.size() - k0);
      cq.push_back((int32_t)qi.size());
      ck.push_back((int32_t)ki.size());
      mq = lq > mq ? lq : mq;
      mk = lk > mk ? lk : mk;
    }
  }
  const int n = (int)cq.size() - 1;
  *num_segments = n;
  *Tq = (int)qi.size();
  *Tk = (int)ki.size();
  *max_q = mq;
  *max_k = mk;
  if (n > max_segments || (n > 0 && (!q_index || !k_index || !cu_q || !cu_k))) {
    vca::set_last_error("attn_ring_segments: max_segments too small, " + std::to_string(n) +
                        " needed");
    return ATTN_E_INVALID;
  }
  for (size_t i = 0; i < qi.size(); ++i) q_index[i] = qi[i];
  for (size_t i = 0; i < ki.size(); ++i) k_index[i] = ki[i];
  for (int i = 0; i <= n && cu_q && cu_k; ++i) {
    cu_q[i] = cq[i];
    cu_k[i] = ck[i];
  }
  return ATTN_OK;
}

// In-place merge of a chunk's live rows versus scatter + dense merge ("gemma4_moe
// cp_attention" page: true when the live-token subset is small enough for
// in-place updates to beat scatter). The pages give no threshold; this compares
// the HBM bytes of the two routes with this library's kernels:
//   in place: per live row, read the fp32 accumulator row and lse, the chunk's
//             row and lse, write the accumulator row and lse, read its index;
//   scatter:  fill the [B, H, S, D] chunk tensor and its lse, write the live
//             rows into it, then merge every one of the B*S rows densely.
extern "C" int attn_ring_inplace_preferred(int64_t live_rows, int64_t B, int64_t S, int H, int D,
                                           int dtype) {
  if (live_rows < 0 || B < 0 || S < 0 || H <= 0 || D <= 0) return 0;
  const int64_t es = dtype == ATTN_F32 ? 4 : 2;  // chunk output element bytes
  const int64_t row_in_place = (int64_t)H * (D * (4 + es + 4) + 4 * 3) + 4;
  const int64_t row_dense = (int64_t)H * (D * (4 + es + 4) + 4 * 3);
  const int64_t scatter = B * S * (int64_t)H * (D * es + 4) + live_rows * (int64_t)H * (D * 2 * es + 8);
  return live_rows * row_in_place < scatter + B * S * row_dense ? 1 : 0;
}
