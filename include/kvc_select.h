/*
 * kvc_select.h -- service-aware choice of a compression profile for each
 * request, from measured profiles.  Host only: no GPU, no device memory.
 *
 * Follows "KVServe: Service-Aware KV Cache Compression for Communication-
 * Efficient Disaggregated LLM Serving":
 *   Sec. 3.1   profile p = (cr_p, s_p, q_p); s_p is the harmonic combination
 *              of the encode and decode throughputs, so that V / s_p is the
 *              total encode + decode time of V bytes;
 *   Sec. 3.2   Eq. 1, request completion time
 *                T_p = T_model + V / s_p + V / (B cr_p),   T_0 = T_model + V / B
 *              (T_0: the KV moved uncompressed); Eq. 2-3, the feasible set
 *              (T_p <= T_SLO, quality bucket) and the arg-min over it;
 *   Sec. 6.1   Eq. 5 / Theorem 6.1: p beats moving raw KV iff
 *              B < B*_p = (1 - 1/cr_p) s_p;
 *              Eq. 6 / Theorem 6.2: with x = 1/B, (T_p - T_model) / V =
 *              1/s_p + x/cr_p is a line, and the optimal profile follows the
 *              lower envelope of the lines: piecewise constant in x;
 *   Sec. 6.2   candidate set = the envelope's optimal profile for the interval
 *              of x plus its envelope neighbours; per (bucket, interval)
 *              environment an EWMA of the residual observed - predicted (Eq. 7)
 *              corrects the prediction (Eq. 8); epsilon-greedy choice among the
 *              candidates; guardrails: predicted T <= T_SLO, a fallback when
 *              nothing is feasible, and a cooldown for a profile with more than
 *              K SLO violations in its last M uses.
 *
 * Readings where the page leaves a step open (the oracle takes the same):
 *   - The uncompressed transfer is itself a line of the envelope (intercept 0,
 *     slope 1, id KVC_PROFILE_RAW), so Theorem 6.1's filter and Theorem 6.2's
 *     envelope are one structure: a profile appears on the envelope only where
 *     it beats raw transfer and every other profile of its bucket.
 *   - Envelope intervals are closed on the left: at a breakpoint the profile
 *     of the next interval is optimal.  Equal lines keep the lowest id.
 *   - The candidate set is the interval's profile plus the profiles of the
 *     adjacent envelope intervals (one or two of them), in envelope order.
 *   - Residual estimates start at 0 and Eq. 7 is applied from the first
 *     observation; an environment is the pair (bucket, envelope interval of
 *     the request's bandwidth).
 *   - Exploration draws: the k-th choose call (k = 0, 1, ...) uses outputs
 *     2k and 2k + 1 of splitmix64 seeded with `seed`.  It explores when at
 *     least two candidates are feasible and (out_2k >> 11) * 2^-53 < epsilon,
 *     and then takes candidate out_{2k+1} mod n of the n feasible candidates
 *     other than the greedy one (in envelope order).  The greedy choice is the
 *     lowest corrected prediction, ties to the earlier envelope position.
 *   - A use is an SLO violation when the observed time exceeds T_SLO.  When a
 *     profile's violations among its last M uses exceed K it sits out the next
 *     `cooldown_len` choose calls and its use history is cleared.  Cooldowns
 *     are per profile, across environments.
 *
 * Selectors are not thread-safe; calls on one selector must not overlap.
 */
#ifndef KVC_SELECT_H
#define KVC_SELECT_H

#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_PROFILE_RAW (-1)   /* moving the KV uncompressed: cr = 1, no codec time */

/* A measured profile.  ids are >= 0 and unique; cr >= 1; throughputs in
 * bytes per second, > 0 and finite. */
typedef struct {
  int32_t id;
  int32_t bucket;     /* quality bucket; profiles are compared within a bucket */
  double cr;          /* V / V_p */
  double s_enc;       /* encode throughput */
  double s_dec;       /* decode throughput */
} kvc_profile;

typedef struct {
  uint32_t struct_size;  /* sizeof(kvc_selector_config) */
  int32_t fallback_id;   /* chosen when no candidate is feasible: a profile id or KVC_PROFILE_RAW */
  double alpha;          /* EWMA weight, in (0, 1] */
  double epsilon;        /* exploration probability, in [0, 1] */
  int32_t cooldown_k;    /* more than K violations ... (>= 0) */
  int32_t cooldown_m;    /* ... among the last M uses (1..64) */
  int32_t cooldown_len;  /* choose calls a profile then sits out (>= 0) */
  int32_t reserved;
  uint64_t seed;         /* exploration draws (splitmix64) */
} kvc_selector_config;

typedef struct {
  int32_t bucket;
  int32_t reserved;
  double bandwidth;      /* B, effective bytes per second, > 0 */
  double volume;         /* V, uncompressed bytes to move, >= 0 */
  double t_model;        /* T_model(w), seconds */
  double t_slo;          /* T_SLO, seconds */
} kvc_request_context;

typedef struct kvc_selector_s* kvc_selector_t;

/* Sec. 3.1: s_enc s_dec / (s_enc + s_dec); 0 if an argument is not > 0. */
double kvc_harmonic_throughput(double s_enc, double s_dec);

/* Eq. 5: (1 - 1/cr) * s_p; 0 if cr < 1 or a throughput is not > 0. */
double kvc_break_even_bandwidth(double cr, double s_enc, double s_dec);

/* Eq. 1 for profile p (NULL: raw transfer, T_model + V / B).  Returns
 * KVC_ERR_INVALID_ARG for NULL c / out or a bandwidth that is not > 0. */
kvc_status kvc_predicted_jct(const kvc_profile* p, const kvc_request_context* c, double* out);

/* Copies the n profiles and the configuration; builds each bucket's lower
 * envelope (Theorem 6.2).  KVC_ERR_INVALID_ARG for bad values or duplicate
 * ids, KVC_ERR_NO_MEMORY if allocation fails. */
kvc_status kvc_selector_create(const kvc_profile* profiles, int32_t n, const kvc_selector_config* cfg,
                               kvc_selector_t* out);
kvc_status kvc_selector_destroy(kvc_selector_t s);

/* The lower envelope of bucket `bucket` (raw transfer included): profile
 * ids[i] is optimal for x = 1/B in [x_from[i], x_from[i + 1]) and the last one
 * for every larger x; x_from[0] = 0.  *count receives the number of
 * intervals; at most `capacity` entries are written (KVC_ERR_BUFFER_TOO_SMALL
 * if capacity < *count).  A bucket without profiles has the single interval
 * of raw transfer. */
kvc_status kvc_selector_envelope(kvc_selector_t s, int32_t bucket, int32_t capacity, int32_t* ids,
                                 double* x_from, int32_t* count);

/* Theorem 6.2 lookup: the envelope's profile for bandwidth B (> 0). */
kvc_status kvc_selector_model_choice(kvc_selector_t s, int32_t bucket, double bandwidth, int32_t* id);

/* Sec. 6.2: choose the profile for one request.  *id receives the choice
 * (KVC_PROFILE_RAW for uncompressed transfer), *predicted_jct (may be NULL)
 * its Eq. 1 prediction.  Advances the exploration counter and the cooldown
 * clock. */
kvc_status kvc_selector_choose(kvc_selector_t s, const kvc_request_context* c, int32_t* id,
                               double* predicted_jct);

/* Report the observed completion time of a request made with profile id under
 * context c: updates the environment's residual (Eq. 7) and use count, and
 * the profile's violation history.  KVC_ERR_INVALID_ARG for an unknown id. */
kvc_status kvc_selector_observe(kvc_selector_t s, const kvc_request_context* c, int32_t id, double observed_jct);

/* Inspection: the residual estimate and use count of profile id in the
 * environment of context c, and the choose calls it still sits out. */
kvc_status kvc_selector_state(kvc_selector_t s, const kvc_request_context* c, int32_t id, double* residual,
                              int64_t* uses, int32_t* cooldown_left);

#ifdef __cplusplus
}
#endif

#endif
