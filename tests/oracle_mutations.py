"""Mutation check of the CPU oracle's pins (run by hand, not collected by pytest).

    python tests/oracle_mutations.py [name ...]

Each entry below plants one plausible mistake in oracle/oracle.c (a dropped
or shifted term, a wrong order, comparison or rounding, a transposed
index, an unguarded bound), builds that copy with the oracle's own compiler
flags into a temporary directory, and runs the CPU suite against it through
MEP_ORACLE_LIB. Every mistake must make at least one test fail; the script
exits non-zero if any survives. The in-tree oracle library is not touched.
The one test that rebuilds the oracle from its source is deselected, since
it would replace the planted build.
"""
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact text in oracle.c, replacement); each text occurs once.
MUTATIONS = [
    ('plan.home',
     '((int64_t)e * (int64_t)R) / (int64_t)E',
     '((int64_t)e * (int64_t)R + 1) / (int64_t)E'),
    ('plan.keep',
     'if (q < C) {',
     'if (q + 1 < C) {'),
    ('plan.spill_desc',
     'for (int u = 0; u < R; u++) {\n            for (int64_t slot = L[u]',
     'for (int u = R - 1; u >= 0; u--) {\n            for (int64_t slot = L[u]'),
    ('plan.zero_redundant',
     'if (home_rank(e, R, E) == u || rcount[(int64_t)u * E + e] == 0) continue;',
     'if (home_rank(e, R, E) == u) continue;'),
    ('plan.send_order',
     'tmp[i].b = route_slot[f];',
     'tmp[i].b = i;'),
    ('plan.recv_order',
     'tmp[t].b = t;',
     'tmp[t].b = -t;'),
    ('plan.gid',
     'gid += n;',
     'gid += n + 1;'),
    ('plan.unstable',
     'order[f].b = f;',
     'order[f].b = N - f;'),
    ('remap.floor',
     'int mode_value = (world_size + count - 1) / count;',
     'int mode_value = world_size / count;'),
    ('remap.mode1_shift',
     'col = t % count + 1;',
     'col = (t + 1) % count + 1;'),
    ('remap.mode1_k',
     'col = t % count + 1;',
     'col = (t * K + k) % count + 1;'),
    ('prune.tie',
     '!(s[k] < thr_sum)',
     '!(s[k] <= thr_sum)'),
    ('prune.fp64',
     'float thr_sum = 0.0f;',
     'double thr_sum = 0.0;'),
    ('prune.reverse',
     'for (int k = 0; k < K; k++) {\n            float prod = s[k] * thr[k];',
     'for (int k = K - 1; k >= 0; k--) {\n            float prod = s[k] * thr[k];'),
    ('prune.fma',
     'float prod = s[k] * thr[k];\n            thr_sum = thr_sum + prod;',
     'thr_sum = fmaf(s[k], thr[k], thr_sum);'),
    ('prune.active',
     'int act = active == NULL ? 1 : (active[t] != 0);',
     'int act = 1;'),
    ('remap.sendmap_inst',
     'tmp[n].a = (int64_t)card * n_inst + inst;',
     'tmp[n].a = (int64_t)card;'),
    ('remap.sendmap_card',
     'int card = inst / place_per_rank;',
     'int card = inst % world_size;'),
    ('fp16.subnormal',
     '127 - 15 - shift + 1',
     '127 - 15 - shift'),
    ('pack.flip',
     'send_buf[(int64_t)row * H + h] = x[t * H + h];',
     'send_buf[(int64_t)row * H + h] = x[t * H + (H - 1 - h)];'),
    ('group.flip',
     'recv_grouped[t * H + h] = recv_raw[src * H + h];',
     'recv_grouped[t * H + h] = recv_raw[src * H + (H - 1 - h)];'),
    ('combine.fma',
     'float y = bf16_to_float(y_ret[(int64_t)row * H + h]);\n                float prod = scores[t * K + k] * y;\n                acc = acc + prod;',
     'float y = bf16_to_float(y_ret[(int64_t)row * H + h]);\n                acc = fmaf(scores[t * K + k], y, acc);'),
    ('combine.reverse',
     'for (int k = 0; k < K; k++) {\n                int32_t row = send_pos[t * K + k];\n                if (row < 0) continue;',
     'for (int k = K - 1; k >= 0; k--) {\n                int32_t row = send_pos[t * K + k];\n                if (row < 0) continue;'),
    ('combine.fp64',
     'float y = bf16_to_float(y_ret[(int64_t)row * H + h]);\n                float prod = scores[t * K + k] * y;\n                acc = acc + prod;',
     'float y = bf16_to_float(y_ret[(int64_t)row * H + h]);\n                float prod = scores[t * K + k] * y;\n                acc = (float)((double)acc + (double)scores[t * K + k] * (double)y); (void)prod;'),
    ('bf16.round_half_up',
     'u += 0x7fffu + lsb;',
     'u += 0x8000u + 0 * lsb;'),
    ('bf16.nan',
     'return (uint16_t)((u >> 16) | 0x0040u);',
     'return (uint16_t)(u >> 16);'),
    ('norm.eps_outside',
     'double r = 1.0 / sqrt(ss / (double)H + eps);',
     'double r = 1.0 / (sqrt(ss / (double)H) + eps);'),
    ('norm.mean_h1',
     'double r = 1.0 / sqrt(ss / (double)H + eps);',
     'double r = 1.0 / sqrt(ss / (double)(H > 1 ? H - 1 : 1) + eps);'),
    ('norm.no_gamma',
     'y[t * H + h] = (double)xs[h] * r * (double)bf16_to_float(gamma[h]);',
     'y[t * H + h] = (double)xs[h] * r;'),
    ('norm.residual_sign',
     'float x = acc + bf16_to_float(residual[t * H + h]);',
     'float x = acc - bf16_to_float(residual[t * H + h]);'),
    ('norm.rounded_x',
     'ss += (double)x * (double)x;',
     'ss += (double)float_to_bf16_rne(x) * 0 + (double)bf16_to_float(float_to_bf16_rne(x)) * (double)bf16_to_float(float_to_bf16_rne(x));'),
    ('quant.128',
     'const float sc = amax / 127.0f;',
     'const float sc = amax / 128.0f;'),
    ('quant.trunc',
     'q = rintf(v[h] / sc);',
     'q = truncf(v[h] / sc);'),
    ('quant.round_away',
     'q = rintf(v[h] / sc);',
     'q = roundf(v[h] / sc);'),
    ('quant.mul_recip',
     'q = rintf(v[h] / sc);',
     'q = rintf(v[h] * (1.0f / sc));'),
    ('quant.scale_pos',
     'memcpy(out + hq, &sc, 4);',
     'memcpy(out + H, &sc, 4);'),
    ('quant.smooth_col',
     'if (smooth) a = a * smooth[(int64_t)e * H + h];',
     'if (smooth) a = a * smooth[(int64_t)e * H];'),
    ('gquant.scale_pos',
     'memcpy(scales + t, m + hq, 4);',
     'memcpy(scales + t, m + H, 4);'),
    ('wrow.le',
     '*out = j < B ? E + j : e;',
     '*out = j <= B ? E + j : e;'),
    ('wrow.reverse',
     '*out = j < B ? E + j : e;',
     '*out = j < B ? E + B - 1 - j : e;'),
    ('wrow.natives_count',
     '*out = e;\n            } else {',
     '*out = e;\n                j++;\n            } else {'),
    ('dedup.reverse_tokens',
     'dpack_pos[t * K + k] = (int32_t)(base[d] + next[d]++);',
     'dpack_pos[t * K + k] = (int32_t)(base[d] + dsend_count[d] - 1 - next[d]++);'),
    ('dedup.src_desc',
     'for (int src = 0; src < R; src++) {\n        int64_t cnt = 0;',
     'for (int src = R - 1; src >= 0; src--) {\n        int64_t cnt = 0;'),
    ('push.flip',
     'grouped[((int64_t)d * C + s) * H + h] = x[t * H + h];',
     'grouped[((int64_t)d * C + s) * H + h] = x[t * H + (H - 1 - h)];'),
    ('pull.fma',
     'float y = bf16_to_float(grouped[((int64_t)d * C + s) * H + h]);\n                float prod = scores[t * K + k] * y;\n                acc = acc + prod;',
     'float y = bf16_to_float(grouped[((int64_t)d * C + s) * H + h]);\n                acc = fmaf(scores[t * K + k], y, acc);'),
    ('plan.load',
     'for (int e = 0; e < E; e++) L[home_rank(e, R, E)] += cnt[e];',
     'for (int e = 0; e < E; e++) L[home_rank(e, R, E)] += cnt[e] + (e == E - 1);'),
    ('plan.inst_fill',
     'for (int i = n; i < E; i++) ie[i] = -1;',
     'for (int i = n; i < E; i++) ie[i] = 0;'),
    ('plan.cu_fill',
     'for (int i = n + 1; i <= E; i++) cu[i] = (int32_t)C;',
     'for (int i = n + 1; i <= E; i++) cu[i] = 0;'),
    ('plan.send_count',
     'send_count[route_dest[f]]++;',
     'send_count[route_dest[f]] += (i == 0) + 1;'),
    ('plan.recv_count',
     'recv_count[src]++;',
     'recv_count[src] += (t == 0) + 1;'),
    ('plan.gid_base_last',
     'inst_gid_base[R] = (int32_t)gid;',
     'inst_gid_base[R] = (int32_t)gid - 1;'),
    ('remap.col_off',
     'balanced_ids[t * K + k] = eplb_table[(int64_t)e * F + col];',
     'balanced_ids[t * K + k] = eplb_table[(int64_t)e * F + col - (col > 1)];'),
    ('remap.sendcount',
     'send_count[card]++;',
     'send_count[card] += (i == 0) + 1;'),
    ('remap.nomask_active',
     'for (int k = 0; k < K; k++) balanced_mask[t * K + k] = 1;\n            continue;',
     'for (int k = 0; k < K; k++) balanced_mask[t * K + k] = (uint8_t)(t != 0);\n            continue;'),
    ('gquant.shift',
     'memcpy(x_q + t * H, m, (size_t)H);',
     'memcpy(x_q + t * H, m + 1, (size_t)H);'),
    ('wrow.past',
     '*out = -1;\n                continue;',
     '*out = 0;\n                continue;'),
    ('dedup.sendcount',
     'if (first && d >= 0 && d < R) dsend_count[d]++;',
     'if (d >= 0 && d < R) dsend_count[d]++;'),
    ('dedup.recvcount',
     'drecv_count[src] = (int32_t)cnt;',
     'drecv_count[src] = (int32_t)cnt + (src == 0);'),
    ('norm.xf32',
     'if (x_f32) x_f32[t * H + h] = x;',
     'if (x_f32) x_f32[t * H + h] = acc;'),
    ('norm.skip_bound',
     'if (row < 0 || row >= n_y) continue;\n                float prod = scores[t * K + k] * bf16_to_float(y_ret',
     'if (row < 0) continue;\n                float prod = scores[t * K + k] * bf16_to_float(y_ret'),
    ('pull.skip',
     'if (d < 0 || d >= R || s < 0 || s >= C) continue;\n                float y',
     'if (d < 0 || d >= R || s < 0 || s >= C) { acc = acc + 0.0f; }\n                if (d < 0) continue; float y'),
    ('quant.skip_bad_expert',
     'if (smooth && (e < 0 || e >= E)) continue;',
     'if (smooth && (e < 0 || e >= E)) e = 0;'),
    ('quant.amax_signed',
     'const float m = fabsf(a);',
     'const float m = a;'),
    ('ungroup.flip',
     'y_arrival[(int64_t)to * H + h] = y_grouped[t * H + h];',
     'y_arrival[(int64_t)to * H + h] = y_grouped[t * H + (H - 1 - h)];'),
]


def main(argv):
    orig = open(SRC).read()
    only = set(argv)
    survived, results = [], []
    with tempfile.TemporaryDirectory() as tmp:
        for name, old, new in MUTATIONS:
            if only and name not in only:
                continue
            if orig.count(old) != 1:
                raise SystemExit(f"{name}: the text to replace occurs {orig.count(old)} times")
            c_path = os.path.join(tmp, name + ".c")
            so_path = os.path.join(tmp, name + ".so")
            with open(c_path, "w") as f:
                f.write(orig.replace(old, new))
            subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                            "-fPIC", "-shared", "-o", so_path, c_path, "-lm"], check=True)
            env = dict(os.environ, MEP_ORACLE_LIB=so_path)
            r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-q",
                                "-x", "-n", "6", "-p", "no:cacheprovider", "--deselect",
                                "tests/test_abi.py::test_c_consumer_builds"],
                               cwd=ROOT, env=env, capture_output=True, text=True)
            failed = [l.split()[1] for l in r.stdout.splitlines() if l.startswith("FAILED")]
            caught = r.returncode != 0 and bool(failed)
            results.append((name, caught, failed[:1]))
            print(f"{name}: {'caught by ' + failed[0] if caught else 'SURVIVED'}", flush=True)
            if not caught:
                survived.append(name)
    print(f"{len(results) - len(survived)} of {len(results)} planted mistakes caught")
    return 1 if survived else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
