"""Host replay of the global-memory index arithmetic of the chunked decode
kernel (window + cache > 128 keys) for sequences at different positions: the
configuration kept off the GPU after two memory faults whose cause was not
found (lengths 192 / 100 / 230, eta = 96, lambda = 64, 3 sequences x 2 KV
heads x 4 query heads, d = 128, bf16, 24 steps, both read orders; decode
refuses it with UNSUPPORTED).

Every load and store of decode_kernel<BF16, 128, true> (keys, value rows,
SRE values, W^T, queries, the leaving and new pairs, s, cache positions,
H, outputs, ring and cache slots, positions) is modelled with the kernel's
own index expressions, per unit, thread and key chunk, and checked against
the element count of its buffer; the LDS tile and SRE-part indices against
the layout.  This is a model kept by hand next to csrc/decode.hip, not the
kernel: it found no access out of bounds.
"""

HD, kM, kD, WP = 128, 64, 128, 8
kThreads, kWaves, kKC, kPend = 256, 4, 128, 3
PER = 8                      # bf16 elements per 16-byte piece
PPR = HD // PER              # 16 pieces per row
CPL = HD // 64               # 2
WPT = kM * PPR // kThreads   # 4
MISC = 8 * PPR + kD // 4     # 160
MPT = (MISC + kThreads - 1) // kThreads
NVS, NS, KB = 5, HD // 32, HD // 32

def run(B, Hkv, g, lam, eta, npos, phase, fails):
    U = B * Hkv
    size = dict(q=U * g * HD, k=U * HD, v=U * HD, WT=Hkv * kM * HD, H=U * kD * HD, s=U * kD,
                ring_k=U * eta * HD, ring_v=U * eta * HD, cache_k=U * lam * HD,
                cache_v=U * lam * HD, cache_pos=U * lam, out=U * g * HD, npos=2 * B,
                pend=U * kPend * (kD + HD), npend=U)
    def chk(buf, off, n, what):
        if off < 0 or off + n > size[buf]:
            fails.append((buf, off, n, size[buf], what))
    for u in range(U):
        b = u // Hkv
        kvh = u % Hkv
        n = npos[b]
        up, rd = phase != 2, phase != 1
        gs = min(lam, max(0, n - eta))
        has_leave = up and n >= eta
        full = has_leave and gs + 1 > lam
        ncand = gs + 1 if full else 0
        w_len = min(eta, n)
        nko = gs + w_len
        ring0 = (n - w_len) % eta if eta > 0 else 0
        ringn = n % eta if eta > 0 else 0
        nch = max(1, (nko + kKC - 1) // kKC)
        qg, kin, vin = u * g * HD, u * HD, u * HD
        ringk = u * eta * HD; ck = u * lam * HD; sg = u * kD; HT = u * kD * HD
        WTb = kvh * kM * HD
        def key_row(kk, val):
            if kk < gs: return ('cache_v' if val else 'cache_k', ck + kk * HD)
            if kk < nko:
                slot = ring0 + (kk - gs)
                if slot >= eta: slot -= eta
                return ('ring_v' if val else 'ring_k', ringk + slot * HD)
            return ('v' if val else 'k', vin if val else kin)
        leave = ('ring', ringk + ringn * HD) if eta > 0 else None
        for tid in range(kThreads):
            lane, wave = tid & 63, tid >> 6
            n16, q4 = lane & 15, lane >> 4
            # npos
            chk('npos', b, 1, 'npos')
            # first wave: keys
            kn0 = min(kKC, nko)
            def kkey(kt, r):                       # block kt of wave w: keys 16 (4 kt + w) ..
                return 16 * (4 * kt + wave) + r
            def load_keys(k0, kn, ln):
                if 16 * wave < kn:
                    for kt in range(2):
                        buf, off = key_row(k0 + min(kkey(kt, ln & 15), kn - 1), False)
                        off += 8 * (ln >> 4)
                        for kb in range(KB): chk(buf, off + 32 * kb, 8, 'keys')
            def load_vals(k0, kn, ln):
                if 16 * wave < kn:
                    for j in range(32):
                        buf, off = key_row(k0 + min(kkey((j >> 4) & 1, j & 15), kn - 1), True)
                        chk(buf, off + CPL * ln, CPL, 'vals')
            def load_vs(row0, rr):
                buf, off = key_row(min(row0 + rr, ncand - 1), True)
                off += 32 * wave + 4 * q4
                for mb in range(2): chk(buf, off + 16 * mb, 4, 'vs')
            load_keys(0, kn0, lane)
            for j in range(WPT):
                i = j * kThreads + tid
                chk('WT', WTb + (i // PPR) * HD + (i % PPR) * PER, PER, 'WT')
            for j in range(MPT):
                i = j * kThreads + tid
                if i < 4 * PPR:
                    if i // PPR < g: chk('q', qg + (i // PPR) * HD + (i % PPR) * PER, PER, 'q')
                elif i < 6 * PPR:
                    if has_leave:
                        base = leave[1] if eta > 0 else kin
                        chk('ring_k' if i < 5 * PPR else 'ring_v', base + (i % PPR) * PER, PER, 'leave')
                elif i < 8 * PPR:
                    chk('k' if i < 7 * PPR else 'v', kin + (i % PPR) * PER, PER, 'new')
                elif i < MISC:
                    chk('s', sg + 4 * (i - 8 * PPR), 4, 's')
            if tid < gs: chk('cache_pos', u * lam + tid, 1, 'cpos')
            for i in range(tid + kThreads, gs, kThreads): chk('cache_pos', u * lam + i, 1, 'cpos2')
            # second wave
            load_vals(0, kn0, lane)
            for t in range(NVS):
                if wave < NS and 16 * t < ncand: load_vs(16 * t, n16)
            if wave < NS:
                for mb in range(2):
                    hrow = HT + (32 * wave + 16 * mb + n16) * kD + 4 * q4
                    for kb in range(4):
                        chk('H', hrow + 32 * kb, 4, 'H'); chk('H', hrow + 32 * kb + 16, 4, 'H')
            for c in range(nch):
                k0 = c * kKC
                kn = max(0, min(kKC, nko - k0))
                last = c == nch - 1
                if c > 0:
                    load_keys(k0, kn, lane); load_vals(k0, kn, lane)
                    for tt in range(NVS):
                        if wave < NS and k0 + 16 * tt < ncand: load_vs(k0 + 16 * tt, lane & 15)
                cno = max(0, min(kn, ncand - k0))
                cn = cno + (1 if (last and ncand > nko) else 0)
                nr = cn + (g if last else 0)
                nt = (nr + 15) // 16
                if nt > 9: fails.append(('slot', nt, 9, 0, 'ntile'))
                if wave < NS:
                    for t in range(NVS, nt):
                        if 16 * t < cn: load_vs(k0 + 16 * t, n16)
                    for t in range(min(NVS, nt)):
                        row = 16 * t + n16
                        if row < cn and k0 + row > lam: fails.append(('spart', k0 + row, lam + 1, 0, 'spart'))
            # outputs
            if wave != 0:
                for i in range(tid - 64, g * HD, kThreads - 64):
                    hd, e = i // HD, i % HD
                    if rd: chk('out', u * g * HD + hd * HD + e, 1, 'out')
                if eta > 0 and up:
                    for i in range(tid - 64, 2 * PPR, kThreads - 64):
                        kk = (i % PPR) * PER
                        chk('ring_k' if i < PPR else 'ring_v', ringk + ringn * HD + kk, PER, 'ringw')
            if wave == 0 and full:
                # argmin over ncand, bi < ncand; value row read bi < gs -> cache
                for bi in range(ncand):
                    if bi != gs: chk('cache_v', ck + bi * HD, HD, 'vrow'); chk('cache_k', ck + bi * HD, HD, 'xrow')
            fold_row_range = range(ncand) if full else [-1]
            for fold_row in fold_row_range:
                if fold_row >= 0:
                    if wave < NS:
                        for mb in range(2):
                            hrow = HT + (32 * wave + 16 * mb + n16) * kD + 4 * q4
                            for kb in range(4): chk('H', hrow + 32 * kb, 4, 'Hw'); chk('H', hrow + 32 * kb + 16, 4, 'Hw')
                    for F in range(tid, kD, kThreads): chk('s', u * kD + F, 1, 'sw')
                if has_leave:
                    slot_in = gs if not full else (fold_row if fold_row < gs else -1)
                    if slot_in >= 0:
                        for i in range(tid, 2 * PPR, kThreads):
                            kk = (i % PPR) * PER
                            chk('cache_k' if i < PPR else 'cache_v', ck + slot_in * HD + kk, PER, 'cw')
                        if tid == 0: chk('cache_pos', u * lam + slot_in, 1, 'cposw')
                if not full: break
            if tid == 0 and u % Hkv == 0: chk('npos', B + b, 1, 'npos_next')  # other half



def test_ragged_chunked_decode_accesses_stay_in_bounds():
    fails = []
    B, Hkv, g, lam, eta = 3, 2, 4, 64, 96
    for order in (0, 1):
        pos = [192, 100, 230]
        for step in range(24):
            if order == 0:
                run(B, Hkv, g, lam, eta, pos, 0, fails)
            else:
                run(B, Hkv, g, lam, eta, pos, 1, fails)
                run(B, Hkv, g, lam, eta, [p + 1 for p in pos], 2, fails)
            pos = [p + 1 for p in pos]
    assert not fails, fails[:10]
