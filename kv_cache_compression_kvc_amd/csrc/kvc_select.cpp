// Service-aware profile selection (host only).  The method is KVServe's
// online controller ("KVServe: Service-Aware KV Cache Compression for
// Communication-Efficient Disaggregated LLM Serving", Sec. 3.1-3.2 and 6);
// the readings taken where the page leaves a step open are listed in
// include/kvc_select.h.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <new>
#include <tuple>
#include <vector>

#include "kvc_select.h"

namespace kvc {
kvc_status report_error(kvc_status s, const char* msg);   // kvc_api.cpp: sets kvc_last_error()
}

namespace {

using kvc::report_error;

// A line y = a + b x of Eq. 6 (x = 1/B, y = (T - T_model) / V).
struct Line {
  int32_t id;
  double a;   // 1 / s_p (0 for raw transfer)
  double b;   // 1 / cr_p (1 for raw transfer)
};

struct Envelope {
  std::vector<Line> seg;       // optimal line per interval, in order of x
  std::vector<double> x_from;  // interval starts; x_from[0] = 0
};

// Lower envelope over x >= 0.  Starting from the line lowest at x = 0, each
// step moves to the line that undercuts the current one first: among the
// lines with a smaller slope, the one whose intersection with the current
// line has the smallest x, ties to the smaller slope (it stays below
// afterwards), then to the lower id.
Envelope build_envelope(std::vector<Line> lines) {
  Envelope e;
  auto lower_at0 = [](const Line& p, const Line& q) {
    if (p.a != q.a) return p.a < q.a;
    if (p.b != q.b) return p.b < q.b;
    return p.id < q.id;
  };
  Line cur = *std::min_element(lines.begin(), lines.end(), lower_at0);
  double x = 0.0;
  e.seg.push_back(cur);
  e.x_from.push_back(0.0);
  for (;;) {
    bool found = false;
    Line best{};
    double bx = 0.0;
    for (const Line& q : lines) {
      if (!(q.b < cur.b)) continue;
      // cur.a + cur.b x = q.a + q.b x
      double xi = (q.a - cur.a) / (cur.b - q.b);
      if (xi < x) xi = x;   // already below (cannot happen after the first step but keeps x monotone)
      if (!found || xi < bx || (xi == bx && (q.b < best.b || (q.b == best.b && (q.a < best.a || (q.a == best.a && q.id < best.id)))))) {
        found = true;
        best = q;
        bx = xi;
      }
    }
    if (!found) break;
    if (bx == x && !e.seg.empty()) {
      // the new line is already optimal where the current interval starts
      e.seg.back() = best;
    } else {
      e.seg.push_back(best);
      e.x_from.push_back(bx);
    }
    cur = best;
    x = bx;
  }
  return e;
}

double harmonic(double s_enc, double s_dec) {
  if (!(s_enc > 0.0) || !(s_dec > 0.0)) return 0.0;
  return s_enc * s_dec / (s_enc + s_dec);
}

// Eq. 1; p == nullptr is raw transfer
double predict(const kvc_profile* p, const kvc_request_context& c) {
  if (!p) return c.t_model + c.volume / c.bandwidth;
  return c.t_model + c.volume / harmonic(p->s_enc, p->s_dec) + c.volume / (c.bandwidth * p->cr);
}

uint64_t splitmix64_at(uint64_t seed, uint64_t k) {
  // output k (0-based) of splitmix64 started at state `seed`
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Arm {         // one profile in one environment
  double residual = 0.0;
  int64_t uses = 0;
};

struct Cool {        // per-profile violation history and cooldown
  uint64_t hist = 0;   // bit i: the (i+1)-th most recent use violated the SLO
  int32_t n = 0;       // uses recorded in hist (<= M)
  int64_t until = 0;   // sits out choose calls with clock < until
};

}  // namespace

struct kvc_selector_s {
  kvc_selector_config cfg;
  std::vector<kvc_profile> prof;             // by index
  std::map<int32_t, size_t> index;           // id -> index into prof
  std::map<int32_t, Envelope> env;           // bucket -> envelope
  std::map<std::tuple<int32_t, int32_t, int32_t>, Arm> arms;   // (bucket, interval, id)
  std::map<int32_t, Cool> cool;              // id (including raw) -> state
  int64_t clock = 0;                         // choose calls so far

  const kvc_profile* find(int32_t id) const {
    auto it = index.find(id);
    return it == index.end() ? nullptr : &prof[it->second];
  }
  const Envelope& envelope(int32_t bucket) {
    auto it = env.find(bucket);
    if (it != env.end()) return it->second;
    return env.emplace(bucket, build_envelope({Line{KVC_PROFILE_RAW, 0.0, 1.0}})).first->second;
  }
  int32_t interval(const Envelope& e, double bandwidth) const {
    const double x = 1.0 / bandwidth;
    // last interval whose start is <= x
    const auto it = std::upper_bound(e.x_from.begin(), e.x_from.end(), x);
    return (int32_t)(it - e.x_from.begin()) - 1;
  }
};

namespace kvc {
// profile lookup for the raw-transfer id: nullptr with ok = true
static bool lookup(const kvc_selector_s* s, int32_t id, const kvc_profile** p) {
  if (id == KVC_PROFILE_RAW) { *p = nullptr; return true; }
  *p = s->find(id);
  return *p != nullptr;
}
}  // namespace kvc

extern "C" {

double kvc_harmonic_throughput(double s_enc, double s_dec) { return harmonic(s_enc, s_dec); }

double kvc_break_even_bandwidth(double cr, double s_enc, double s_dec) {
  const double sp = harmonic(s_enc, s_dec);
  if (!(cr >= 1.0) || sp == 0.0) return 0.0;
  return (1.0 - 1.0 / cr) * sp;
}

kvc_status kvc_predicted_jct(const kvc_profile* p, const kvc_request_context* c, double* out) {
  if (!c || !out) return report_error(KVC_ERR_INVALID_ARG, "kvc_predicted_jct: NULL argument");
  if (!(c->bandwidth > 0.0)) return report_error(KVC_ERR_INVALID_ARG, "kvc_predicted_jct: bandwidth must be > 0");
  if (p && (!(p->cr >= 1.0) || harmonic(p->s_enc, p->s_dec) == 0.0))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_predicted_jct: bad profile");
  *out = predict(p, *c);
  return KVC_OK;
}

kvc_status kvc_selector_create(const kvc_profile* profiles, int32_t n, const kvc_selector_config* cfg,
                               kvc_selector_t* out) {
  if (!cfg || !out || n < 0 || (n > 0 && !profiles))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_create: NULL argument or negative count");
  if (cfg->struct_size != sizeof(kvc_selector_config))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_create: struct_size mismatch");
  if (!(cfg->alpha > 0.0 && cfg->alpha <= 1.0) || !(cfg->epsilon >= 0.0 && cfg->epsilon <= 1.0) ||
      cfg->cooldown_k < 0 || cfg->cooldown_m < 1 || cfg->cooldown_m > 64 || cfg->cooldown_len < 0)
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_create: alpha in (0,1], epsilon in [0,1], "
                                             "cooldown_k >= 0, 1 <= cooldown_m <= 64, cooldown_len >= 0");
  kvc_selector_s* s = new (std::nothrow) kvc_selector_s();
  if (!s) return report_error(KVC_ERR_NO_MEMORY, "kvc_selector_create: out of memory");
  try {
    s->cfg = *cfg;
    std::map<int32_t, std::vector<Line>> lines;
    for (int32_t i = 0; i < n; ++i) {
      const kvc_profile& p = profiles[i];
      const bool finite = std::isfinite(p.cr) && std::isfinite(p.s_enc) && std::isfinite(p.s_dec);
      if (p.id < 0 || !finite || !(p.cr >= 1.0) || !(p.s_enc > 0.0) || !(p.s_dec > 0.0) || s->index.count(p.id)) {
        delete s;
        return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_create: profile ids must be unique and >= 0, "
                                                 "cr >= 1, throughputs finite and > 0");
      }
      s->index[p.id] = s->prof.size();
      s->prof.push_back(p);
      lines[p.bucket].push_back(Line{p.id, 1.0 / harmonic(p.s_enc, p.s_dec), 1.0 / p.cr});
    }
    if (cfg->fallback_id != KVC_PROFILE_RAW && !s->index.count(cfg->fallback_id)) {
      delete s;
      return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_create: fallback_id is not a profile id");
    }
    for (auto& kv : lines) {
      kv.second.push_back(Line{KVC_PROFILE_RAW, 0.0, 1.0});
      s->env.emplace(kv.first, build_envelope(kv.second));
    }
  } catch (const std::bad_alloc&) {
    delete s;
    return report_error(KVC_ERR_NO_MEMORY, "kvc_selector_create: out of memory");
  }
  *out = s;
  return KVC_OK;
}

kvc_status kvc_selector_destroy(kvc_selector_t s) {
  delete s;
  return KVC_OK;
}

kvc_status kvc_selector_envelope(kvc_selector_t s, int32_t bucket, int32_t capacity, int32_t* ids,
                                 double* x_from, int32_t* count) {
  if (!s || !count || capacity < 0 || (capacity > 0 && (!ids || !x_from)))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_envelope: NULL argument");
  const Envelope& e = s->envelope(bucket);
  const int32_t m = (int32_t)e.seg.size();
  *count = m;
  for (int32_t i = 0; i < m && i < capacity; ++i) {
    ids[i] = e.seg[i].id;
    x_from[i] = e.x_from[i];
  }
  if (capacity < m) return report_error(KVC_ERR_BUFFER_TOO_SMALL, "kvc_selector_envelope: capacity < count");
  return KVC_OK;
}

kvc_status kvc_selector_model_choice(kvc_selector_t s, int32_t bucket, double bandwidth, int32_t* id) {
  if (!s || !id || !(bandwidth > 0.0))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_model_choice: NULL argument or bandwidth <= 0");
  const Envelope& e = s->envelope(bucket);
  *id = e.seg[s->interval(e, bandwidth)].id;
  return KVC_OK;
}

kvc_status kvc_selector_choose(kvc_selector_t s, const kvc_request_context* c, int32_t* id,
                               double* predicted_jct) {
  if (!s || !c || !id || !(c->bandwidth > 0.0))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_choose: NULL argument or bandwidth <= 0");
  const Envelope& e = s->envelope(c->bucket);
  const int32_t i = s->interval(e, c->bandwidth);
  const int64_t k = s->clock++;
  // candidates: the interval's profile and its envelope neighbours, in envelope order
  struct Cand { int32_t id; double pred; double eff; };
  std::vector<Cand> feas;
  for (int32_t j = std::max(0, i - 1); j <= std::min((int32_t)e.seg.size() - 1, i + 1); ++j) {
    const int32_t pid = e.seg[j].id;
    const auto ct = s->cool.find(pid);
    if (ct != s->cool.end() && k < ct->second.until) continue;           // cooling down
    const kvc_profile* p = nullptr;
    kvc::lookup(s, pid, &p);
    const double pred = predict(p, *c);
    if (!(pred <= c->t_slo)) continue;                                    // guardrail
    double res = 0.0;
    const auto at = s->arms.find(std::make_tuple(c->bucket, i, pid));
    if (at != s->arms.end()) res = at->second.residual;
    feas.push_back(Cand{pid, pred, pred + res});                          // Eq. 8
  }
  if (feas.empty()) {
    const kvc_profile* p = nullptr;
    kvc::lookup(s, s->cfg.fallback_id, &p);
    *id = s->cfg.fallback_id;
    if (predicted_jct) *predicted_jct = predict(p, *c);
    return KVC_OK;
  }
  size_t g = 0;
  for (size_t j = 1; j < feas.size(); ++j)
    if (feas[j].eff < feas[g].eff) g = j;
  size_t pick = g;
  if (feas.size() >= 2) {
    const uint64_t u = splitmix64_at(s->cfg.seed, 2 * (uint64_t)k);
    if ((double)(u >> 11) * 0x1.0p-53 < s->cfg.epsilon) {
      const uint64_t r = splitmix64_at(s->cfg.seed, 2 * (uint64_t)k + 1);
      size_t nth = (size_t)(r % (uint64_t)(feas.size() - 1));
      pick = nth < g ? nth : nth + 1;                                     // skip the greedy one
    }
  }
  *id = feas[pick].id;
  if (predicted_jct) *predicted_jct = feas[pick].pred;
  return KVC_OK;
}

kvc_status kvc_selector_observe(kvc_selector_t s, const kvc_request_context* c, int32_t id, double observed_jct) {
  if (!s || !c || !(c->bandwidth > 0.0))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_observe: NULL argument or bandwidth <= 0");
  const kvc_profile* p = nullptr;
  if (!kvc::lookup(s, id, &p)) return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_observe: unknown profile id");
  const Envelope& e = s->envelope(c->bucket);
  const int32_t i = s->interval(e, c->bandwidth);
  Arm& a = s->arms[std::make_tuple(c->bucket, i, id)];
  const double delta = observed_jct - predict(p, *c);
  a.residual = (1.0 - s->cfg.alpha) * a.residual + s->cfg.alpha * delta;   // Eq. 7
  a.uses += 1;
  Cool& h = s->cool[id];
  const uint64_t keep = s->cfg.cooldown_m == 64 ? ~0ull : ((1ull << s->cfg.cooldown_m) - 1);
  h.hist = ((h.hist << 1) | (observed_jct > c->t_slo ? 1ull : 0ull)) & keep;
  h.n = std::min(h.n + 1, s->cfg.cooldown_m);
  if (__builtin_popcountll(h.hist) > s->cfg.cooldown_k) {
    h.until = s->clock + s->cfg.cooldown_len;
    h.hist = 0;
    h.n = 0;
  }
  return KVC_OK;
}

kvc_status kvc_selector_state(kvc_selector_t s, const kvc_request_context* c, int32_t id, double* residual,
                              int64_t* uses, int32_t* cooldown_left) {
  if (!s || !c || !(c->bandwidth > 0.0))
    return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_state: NULL argument or bandwidth <= 0");
  const kvc_profile* p = nullptr;
  if (!kvc::lookup(s, id, &p)) return report_error(KVC_ERR_INVALID_ARG, "kvc_selector_state: unknown profile id");
  const Envelope& e = s->envelope(c->bucket);
  const int32_t i = s->interval(e, c->bandwidth);
  const auto at = s->arms.find(std::make_tuple(c->bucket, i, id));
  if (residual) *residual = at == s->arms.end() ? 0.0 : at->second.residual;
  if (uses) *uses = at == s->arms.end() ? 0 : at->second.uses;
  if (cooldown_left) {
    const auto ct = s->cool.find(id);
    *cooldown_left = ct == s->cool.end() ? 0 : (int32_t)std::max<int64_t>(0, ct->second.until - s->clock);
  }
  return KVC_OK;
}

}  // extern "C"
