"""Writes silu_decimal.json: SiLU(x) = x / (1 + e^{-x}) at 50 significant digits,
computed with Python's decimal module (correctly rounded exp).  Uses neither the
oracle nor the HIP library.  SiLU is named (as Swish) on "GEMM o Coração
Matemático" §13.3 and "Resumo Técnico: Sobreposição de Ativação em Nível de Tile
para Inferência Eficiente de LLM" (Metodologia/Kernel-1); the formula is the
standard one (Swish with unit slope)."""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 50
POINTS = ["-30", "-10", "-2.5", "-1", "-0.5", "-0.0078125", "0", "0.0078125", "0.25",
          "0.5", "1", "1.5", "2", "3", "8", "20", "40"]


def silu(x: Decimal) -> Decimal:
    return x / (1 + (-x).exp())


out = {"source": __doc__.strip().splitlines()[0],
       "digits": 50,
       "values": [{"x": p, "silu": str(silu(Decimal(p)))} for p in POINTS]}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "silu_decimal.json"), "w") as f:
    json.dump(out, f, indent=1)
